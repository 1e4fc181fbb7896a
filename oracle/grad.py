"""Gradients of the selective scan (test infrastructure only).

Only the tests and the benchmark's CPU-baseline leg may import this module.
The pages pin the backward pass only as automatic differentiation of the
scan loop (Vision Mamba page, the reference loop of implementation row 4 and
its training setting), so the oracle is exactly that: the loop of "A state
retains, writes, and reads" written with plain PyTorch CPU operations in
float64, differentiated by torch.autograd.  The forward arithmetic follows
the C oracle's order (flip, scan, flip for the reverse direction) so that the
two forwards agree to rounding; tests pin the gradients to central finite
differences of the C oracle.
"""
from __future__ import annotations

import numpy as np
import torch

_F = torch.float64


def _t(a, grad=True):
    if a is None:
        return None
    t = torch.tensor(np.asarray(a, dtype=np.float64), dtype=_F)
    return t.requires_grad_(grad)


def _scan_loop(u, delta, A, B, C, D, bias, delta_softplus):
    """y[b, d, t] of one forward scan from a zero state (plain loop over t)."""
    batch, dim, L = u.shape
    N = A.shape[1]
    x = delta + (bias[None, :, None] if bias is not None else 0.0)
    # softplus without torch's large-argument shortcut, so it is log(1 + e^x)
    # everywhere (the test ranges keep e^x finite)
    dt = torch.nn.functional.softplus(x, threshold=1e30) if delta_softplus else x
    h = torch.zeros((batch, dim, N), dtype=_F)
    ys = []
    for t in range(L):
        a = torch.exp(dt[:, :, t, None] * A[None, :, :])
        h = a * h + dt[:, :, t, None] * B[:, None, :, t] * u[:, :, t, None]
        ys.append((C[:, None, :, t] * h).sum(-1) + D[None, :] * u[:, :, t])
    return torch.stack(ys, dim=-1)


def _direction_y(p, delta_softplus, reverse):
    u, dl, A, B, C, D, bias = p
    if reverse:
        f = lambda v: torch.flip(v, dims=[-1])
        return f(_scan_loop(f(u), f(dl), A, f(B), f(C), D, bias, delta_softplus))
    return _scan_loop(u, dl, A, B, C, D, bias, delta_softplus)


_KEYS = ("u", "delta", "A", "B", "C", "D", "delta_bias")


def _leaves(p):
    return [_t(p.get(k)) for k in _KEYS]


def _grads(leaves):
    return {k: (None if v is None else v.grad.numpy().copy()) for k, v in zip(_KEYS, leaves)}


def selective_scan_grad(p, dout, z=None, delta_softplus=True, reverse=False):
    """Gradients of L = sum(dout * out) for out = y * SiLU(z) (y without z).
    p: dict u, delta, A, B, C, D, delta_bias (numpy, the forward's shapes).
    Returns (grads dict with the keys of p, dz or None, out)."""
    lv = _leaves(p)
    zt = _t(z)
    y = _direction_y(lv, delta_softplus, reverse)
    out = y * torch.nn.functional.silu(zt) if zt is not None else y
    (out * _t(dout, False)).sum().backward()
    return _grads(lv), (zt.grad.numpy().copy() if zt is not None else None), out.detach().numpy()


def bidir_scan_grad(fwd, bwd, dout, z=None, combine_scale=1.0, delta_softplus=True):
    """Gradients of L = sum(dout * out), out = s * (y_f + flip(scan(flip(bwd)))) * SiLU(z).
    Returns (grads of fwd, grads of bwd, dz or None, out)."""
    lf, lb = _leaves(fwd), _leaves(bwd)
    zt = _t(z)
    y = combine_scale * (_direction_y(lf, delta_softplus, False) + _direction_y(lb, delta_softplus, True))
    out = y * torch.nn.functional.silu(zt) if zt is not None else y
    (out * _t(dout, False)).sum().backward()
    return _grads(lf), _grads(lb), (zt.grad.numpy().copy() if zt is not None else None), \
        out.detach().numpy()
