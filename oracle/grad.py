"""Gradients of the selective scan (test infrastructure only).

Only the tests and the benchmark's CPU-baseline leg may import this module.
The pages pin the backward pass only as automatic differentiation of the
scan loop (Vision Mamba page, the reference loop of implementation row 4 and
its training setting), so the oracle is exactly that: the loop of "A state
retains, writes, and reads" written with plain PyTorch CPU operations in
float64, differentiated by torch.autograd.  With zoh=True the write uses the
zero-order-hold coefficient of the "Norm or Direction?" page (section 3,
eq. 2) for diagonal A, expm1(dt A) / A per state, in place of dt.  The forward arithmetic follows
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


def _zoh_coef(dt, A):
    """expm1(dt A) / A, written as dt phi(x) with phi(x) = expm1(x) / x and
    x = dt A.  Near x = 0 (A = 0 included, where the coefficient is dt) phi
    is its Taylor series, so that the value and its derivatives stay exact
    there."""
    x = dt * A
    small = x.abs() < 1e-3
    xs = torch.where(small, torch.ones_like(x), x)
    phi = torch.where(small, 1 + x * (1 / 2 + x * (1 / 6 + x * (1 / 24 + x / 120))),
                      torch.expm1(xs) / xs)
    return dt * phi


def _scan_loop(u, delta, A, B, C, D, bias, delta_softplus, zoh=False):
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
        dtt = dt[:, :, t, None]
        a = torch.exp(dtt * A[None, :, :])
        k = _zoh_coef(dtt, A[None, :, :]) if zoh else dtt
        h = a * h + k * B[:, None, :, t] * u[:, :, t, None]
        ys.append((C[:, None, :, t] * h).sum(-1) + D[None, :] * u[:, :, t])
    return torch.stack(ys, dim=-1)


def _direction_y(p, delta_softplus, reverse, zoh=False):
    u, dl, A, B, C, D, bias = p
    if reverse:
        f = lambda v: torch.flip(v, dims=[-1])
        return f(_scan_loop(f(u), f(dl), A, f(B), f(C), D, bias, delta_softplus, zoh))
    return _scan_loop(u, dl, A, B, C, D, bias, delta_softplus, zoh)


_KEYS = ("u", "delta", "A", "B", "C", "D", "delta_bias")


def _leaves(p):
    return [_t(p.get(k)) for k in _KEYS]


def _grads(leaves):
    return {k: (None if v is None else v.grad.numpy().copy()) for k, v in zip(_KEYS, leaves)}


def selective_scan_grad(p, dout, z=None, delta_softplus=True, reverse=False, zoh=False):
    """Gradients of L = sum(dout * out) for out = y * SiLU(z) (y without z).
    p: dict u, delta, A, B, C, D, delta_bias (numpy, the forward's shapes).
    Returns (grads dict with the keys of p, dz or None, out)."""
    lv = _leaves(p)
    zt = _t(z)
    y = _direction_y(lv, delta_softplus, reverse, zoh)
    out = y * torch.nn.functional.silu(zt) if zt is not None else y
    (out * _t(dout, False)).sum().backward()
    return _grads(lv), (zt.grad.numpy().copy() if zt is not None else None), out.detach().numpy()


def bidir_scan_grad(fwd, bwd, dout, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Gradients of L = sum(dout * out), out = s * (y_f + flip(scan(flip(bwd)))) * SiLU(z).
    Returns (grads of fwd, grads of bwd, dz or None, out)."""
    lf, lb = _leaves(fwd), _leaves(bwd)
    zt = _t(z)
    y = combine_scale * (_direction_y(lf, delta_softplus, False, zoh) +
                         _direction_y(lb, delta_softplus, True, zoh))
    out = y * torch.nn.functional.silu(zt) if zt is not None else y
    (out * _t(dout, False)).sum().backward()
    return _grads(lf), _grads(lb), (zt.grad.numpy().copy() if zt is not None else None), \
        out.detach().numpy()


def causal_conv1d_silu_grad(x, w, bias, du, reverse=False):
    """Gradients of L = sum(du * u) for the block's depthwise causal conv of
    width 4 plus bias, then SiLU (Vision Mamba page, "Inside the released Vim
    block"): u[t] = SiLU(bias + sum_k w[k] x[t - 3 + k]), taps before the row
    start reading 0; reverse=True is the backward branch's (flip, convolve,
    flip back).  Returns (dx, dw, dbias or None, u)."""
    xt, wt, bt = _t(x), _t(w), _t(bias)
    f = (lambda v: torch.flip(v, dims=[-1])) if reverse else (lambda v: v)
    xs = f(xt)
    L = xs.shape[-1]
    v = bt[None, :, None].expand(xs.shape[0], -1, L) if bt is not None else torch.zeros_like(xs)
    for k in range(4):
        shift = 3 - k                     # tap k reads x[t - shift]
        if shift >= L:
            continue
        xk = torch.nn.functional.pad(xs[:, :, :L - shift], (shift, 0)) if shift else xs
        v = v + wt[None, :, k, None] * xk
    u = f(torch.nn.functional.silu(v))
    (u * _t(du, False)).sum().backward()
    return xt.grad.numpy().copy(), wt.grad.numpy().copy(), \
        (bt.grad.numpy().copy() if bt is not None else None), u.detach().numpy()


def pool_scan_repeat_grad(fwd, bwd, dout, z=None, combine_scale=1.0, pool_axis=0,
                          delta_softplus=True, zoh=False):
    """Gradients of L = sum(dout * out) for the FastVim pooled path (FastVim
    summary, "Methodology"): u [batch, dim, H, W] is mean-pooled over W
    (pool_axis 0, Lp = H) or over H (axis 1, Lp = W) as (sum in index order)
    times 1/w, the pooled sequence is scanned forward (and backward when bwd
    is given), the sum is repeated along the pooled axis and gated with
    SiLU(z).  delta, B, C have the pooled length.  Returns (grads of fwd,
    grads of bwd or None, dz or None, out)."""
    lf = _leaves(fwd)
    lb = _leaves(bwd) if bwd is not None else None
    zt = _t(z)

    def pooled(lv):
        u = lv[0]
        w = u.shape[3] if pool_axis == 0 else u.shape[2]
        ubar = u.sum(dim=3 if pool_axis == 0 else 2) * (1.0 / w)
        return [ubar] + lv[1:]

    y = _direction_y(pooled(lf), delta_softplus, False, zoh)
    if lb is not None:
        y = y + _direction_y(pooled(lb), delta_softplus, True, zoh)
    rep = y[:, :, :, None] if pool_axis == 0 else y[:, :, None, :]
    out = combine_scale * rep.expand(fwd["u"].shape)
    if zt is not None:
        out = out * torch.nn.functional.silu(zt)
    (out * _t(dout, False)).sum().backward()
    return _grads(lf), (_grads(lb) if lb is not None else None), \
        (zt.grad.numpy().copy() if zt is not None else None), out.detach().numpy()


def ss2d_scan_grad(u, dirs, dout, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Gradients of L = sum(dout * out) for the four-direction 2-D scan
    ("Norm or Direction?" page, section 3, "2D Selective Scan (SS2D)"): the
    map u [batch, dim, H, W] is traversed row-major (k = 0), reversed (1),
    column-major (2) and reversed (3); direction k's delta, B, C follow the
    steps of its base order; the outputs, put back on the map, are summed,
    scaled and gated with SiLU(z).  dirs: four dicts of delta, A, B, C, D,
    delta_bias.  Returns (du, grads per direction without u, dz or None,
    out)."""
    ut = _t(u)
    batch, dim, H, W = ut.shape
    zt = _t(z)
    keys = _KEYS[1:]
    leaves = [[_t(d.get(k)) for k in keys] for d in dirs]
    total = 0.0
    for k, lv in enumerate(leaves):
        seq = (ut if k < 2 else ut.transpose(2, 3)).reshape(batch, dim, H * W)
        y = _direction_y([seq] + lv, delta_softplus, k % 2 == 1, zoh)
        total = total + (y.reshape(batch, dim, H, W) if k < 2 else
                         y.reshape(batch, dim, W, H).transpose(2, 3))
    out = combine_scale * total
    if zt is not None:
        out = out * torch.nn.functional.silu(zt)
    (out * _t(dout, False)).sum().backward()
    grads = [{k: (None if v is None else v.grad.numpy().copy()) for k, v in zip(keys, lv)} for lv in leaves]
    return ut.grad.numpy().copy(), grads, (zt.grad.numpy().copy() if zt is not None else None), \
        out.detach().numpy()

