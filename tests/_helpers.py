"""Shared helpers for the GPU parity tests."""
import numpy as np
import torch

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def rel_err(got, ref, floor_frac=0.1):
    """max_i |got - ref| / max(|ref_i|, floor_frac * rms(ref)); 0/0 := 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    floor = floor_frac * float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), floor)
    num = np.abs(got - ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(num == 0, 0.0, num / den)
    return float(np.max(r))


def host(t):
    """Tensor -> float64 numpy (bf16 and fp32 widen exactly)."""
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


def host_dir(p):
    return {k: host(v) for k, v in p.items()}


def assert_close(got, ref, tol, what=""):
    e = rel_err(got, ref)
    e3 = rel_err(got, ref, 0.01), rel_err(got, ref, 1.0)
    print(f"{what}: rel err (floor 0.1 rms) {e:.3e}; floor 0.01 rms {e3[0]:.3e}; floor rms {e3[1]:.3e}")
    assert np.all(np.isfinite(got)), "non-finite output"
    assert e <= tol, f"{what}: rel err {e:.3e} > {tol:.1e}"


def sub_dir(p, bidx, didx, L=None):
    """Restrict one direction's tensors to batch rows bidx and channels didx
    (rows are independent, so the oracle can check a sample of them)."""
    out = {}
    for k, v in p.items():
        if v is None:
            out[k] = None
        elif k in ("u", "delta"):
            out[k] = v[bidx][:, didx]
        elif k in ("B", "C"):
            out[k] = v[bidx]
        elif k == "A":
            out[k] = v[didx]
        else:                       # D, delta_bias
            out[k] = v[didx]
    return out


def bits_equal(t, ref64):
    """Bitwise equality of a fp32 / bf16 tensor with float64 reference values
    that are exactly representable in its dtype (signed zeros distinguished)."""
    ref = torch.from_numpy(np.ascontiguousarray(ref64)).to(t.dtype)
    if not torch.equal(ref.to(torch.float64), torch.from_numpy(np.ascontiguousarray(ref64))):
        return False                       # reference not representable: not a copy
    ib = torch.int16 if t.dtype == torch.bfloat16 else torch.int32
    return torch.equal(t.detach().cpu().contiguous().view(ib), ref.contiguous().view(ib))
