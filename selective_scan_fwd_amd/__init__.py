"""Selective-scan hot path for vision Mamba backbones on AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/vm_scan.h (libvmscan.so, built
in-tree by ``selective_scan_fwd_amd.build``).  The functions here only check
tensor shapes / dtypes / devices and marshal pointers; every step of the
computation runs in the library's HIP kernels on the current torch stream.
PyTorch supplies device memory and the stream.  There is no fallback: if the
library is missing or fails to load, every call raises.

Names and argument order follow the C ABI:
  vm_selective_scan_fwd, vm_bidir_scan_fwd, vm_atrous_gather,
  vm_atrous_scatter, vm_pool_scan_repeat, vm_ss2d_scan_fwd,
  vm_causal_conv1d_silu, vm_causal_conv1d_silu_bwd, vm_selective_scan_bwd,
  vm_bidir_scan_bwd, vm_pool_scan_repeat_bwd, vm_ss2d_scan_bwd,
  vm_atrous_group_len.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvmscan.so")

VM_F32, VM_BF16 = 0, 1
VM_DELTA_SOFTPLUS, VM_ZOH = 1, 2
VM_OK = 0
STATUS_NAMES = {0: "VM_OK", 1: "VM_ERR_NULL", 2: "VM_ERR_SHAPE", 3: "VM_ERR_DTYPE", 4: "VM_ERR_FLAG",
                5: "VM_ERR_ALIAS", 6: "VM_ERR_UNSUPPORTED", 7: "VM_ERR_HIP", 8: "VM_ERR_ALLOC"}

EXPORTED = ("vm_status_string", "vm_version", "vm_selective_scan_fwd", "vm_bidir_scan_fwd",
            "vm_bidir_scan_fwd_noalloc",
            "vm_atrous_group_len", "vm_atrous_gather", "vm_atrous_scatter", "vm_pool_scan_repeat",
            "vm_ss2d_scan_fwd", "vm_causal_conv1d_silu", "vm_causal_conv1d_silu_bwd",
            "vm_selective_scan_bwd", "vm_bidir_scan_bwd", "vm_pool_scan_repeat_bwd",
            "vm_ss2d_scan_bwd")


class VmScanDir(ctypes.Structure):
    """struct vm_scan_dir (one scan direction's device pointers)."""
    _fields_ = [("u", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("delta_bias", ctypes.c_void_p), ("bc_stride", ctypes.c_int64),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p)]


class VmScanGrad(ctypes.Structure):
    """struct vm_scan_grad (one direction's gradient buffers)."""
    _fields_ = [(k, ctypes.c_void_p) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias",
                                                "dconv_w", "dconv_b")]


class VmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_lock = threading.Lock()
_lib = None


def load_library():
    """Load libvmscan.so and declare the C signatures.  Raises if absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run selective_scan_fwd_amd.build.build() "
                                   "first")
            lib = ctypes.CDLL(LIB_PATH)
            P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
            D = ctypes.POINTER(VmScanDir)
            lib.vm_status_string.argtypes = [I]
            lib.vm_status_string.restype = ctypes.c_char_p
            lib.vm_version.argtypes = []
            lib.vm_version.restype = I
            lib.vm_selective_scan_fwd.argtypes = [D, P, P, I64, I64, I64, I64, I, I, I, P]
            lib.vm_bidir_scan_fwd.argtypes = [D, D, P, F, P, I64, I64, I64, I64, I, I, P]
            lib.vm_bidir_scan_fwd_noalloc.argtypes = [D, D, P, F, P, I64, I64, I64, I64, I, I, P]
            lib.vm_atrous_group_len.argtypes = [I64, I64]
            lib.vm_atrous_group_len.restype = I64
            lib.vm_atrous_gather.argtypes = [P, P, I64, I64, I64, I64, I, P]
            lib.vm_atrous_scatter.argtypes = [P, P, I64, I64, I64, I64, I, P]
            lib.vm_pool_scan_repeat.argtypes = [D, D, P, F, P, I64, I64, I64, I64, I64, I, I, I, P]
            lib.vm_ss2d_scan_fwd.argtypes = [D, P, P, F, P, I64, I64, I64, I64, I64, I, I, P]
            lib.vm_causal_conv1d_silu.argtypes = [P, P, P, P, I64, I64, I64, I, I, P]
            lib.vm_causal_conv1d_silu_bwd.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, I, P]
            G = ctypes.POINTER(VmScanGrad)
            lib.vm_selective_scan_bwd.argtypes = [D, P, P, G, P, I64, I64, I64, I64, I, I, I, P]
            lib.vm_bidir_scan_bwd.argtypes = [D, D, P, P, F, G, G, P, I64, I64, I64, I64, I, I, P]
            lib.vm_pool_scan_repeat_bwd.argtypes = [D, D, P, P, F, G, G, P, I64, I64, I64, I64, I64, I, I, I, P]
            lib.vm_ss2d_scan_bwd.argtypes = [D, P, P, P, F, G, P, P, I64, I64, I64, I64, I64, I, I, P]
            for name in ("vm_selective_scan_fwd", "vm_bidir_scan_fwd", "vm_bidir_scan_fwd_noalloc",
                         "vm_atrous_gather",
                         "vm_atrous_scatter", "vm_pool_scan_repeat", "vm_ss2d_scan_fwd",
                         "vm_causal_conv1d_silu", "vm_causal_conv1d_silu_bwd", "vm_selective_scan_bwd",
                         "vm_bidir_scan_bwd", "vm_pool_scan_repeat_bwd", "vm_ss2d_scan_bwd"):
                getattr(lib, name).restype = I
            _lib = lib
    return _lib


def vm_status_string(status: int) -> str:
    return load_library().vm_status_string(int(status)).decode()


def vm_version() -> int:
    return int(load_library().vm_version())


def _check(status, what):
    if status != VM_OK:
        raise VmError(status, f"{what}: {vm_status_string(status)}")


# ---------------------------------------------------------------- marshalling
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return VM_F32
    if t.dtype == torch.bfloat16:
        return VM_BF16
    raise TypeError(f"token tensors must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _bc(t: torch.Tensor, name: str, dtype, shape, device):
    """B or C [batch, N, L]: dense, or a transposed view of token-major
    [batch, L, >= N] memory.  Returns the C ABI's bc_stride (0 = dense)."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    batch, n, L = shape
    if t.is_contiguous():
        return 0
    sb, sn, st = t.stride()
    if sn == 1 and st >= n and (sb == L * st or batch == 1):
        return st
    raise ValueError(f"{name} must be dense [batch, N, L] or a transposed view of token-major "
                     f"[batch, L, >= N] memory (strides {t.stride()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _options(delta_softplus, zoh):
    return (VM_DELTA_SOFTPLUS if delta_softplus else 0) | (VM_ZOH if zoh else 0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _direction(p, batch, dim, u_shape, tok_len, dstate, dt, device, name):
    """Validate one direction dict and return (VmScanDir, keepalive)."""
    u = _dev(p["u"], f"{name}.u", dt, u_shape, device)
    delta = _dev(p["delta"], f"{name}.delta", dt, (batch, dim, tok_len), device)
    A = _dev(p["A"], f"{name}.A", torch.float32, (dim, dstate), device)
    B, C = p["B"], p["C"]
    sB = _bc(B, f"{name}.B", dt, (batch, dstate, tok_len), device)
    sC = _bc(C, f"{name}.C", dt, (batch, dstate, tok_len), device)
    if sB != sC:
        raise ValueError(f"{name}.B and {name}.C must share one layout (bc strides {sB} vs {sC})")
    D = _dev(p["D"], f"{name}.D", torch.float32, (dim,), device)
    bias = p.get("delta_bias")
    if bias is not None:
        bias = _dev(bias, f"{name}.delta_bias", torch.float32, (dim,), device)
    cw, cb = p.get("conv_w"), p.get("conv_b")
    if cw is not None:
        cw = _dev(cw, f"{name}.conv_w", torch.float32, (dim, 4), device)
        if cb is not None:
            cb = _dev(cb, f"{name}.conv_b", torch.float32, (dim,), device)
    else:
        cb = None
    ptr = lambda t: t.data_ptr() if t is not None else None
    s = VmScanDir(u.data_ptr(), delta.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(),
                  D.data_ptr(), ptr(bias), sB, ptr(cw), ptr(cb))
    return s, (u, delta, A, B, C, D, bias, cw, cb)


# ---------------------------------------------------------------- entry points
def vm_selective_scan_fwd(u, delta, A, B, C, D, z=None, delta_bias=None, delta_softplus=True,
                          reverse=False, out=None, zoh=False, conv_w=None, conv_b=None):
    """One-direction selective scan; returns out shaped like u.
    u, delta, z: [batch, dim, L]; A: [dim, N] fp32; B, C: [batch, N, L]
    (dense, or transposed views of token-major [batch, L, N] memory, which
    the kernels read directly); D, delta_bias: [dim] fp32.
    reverse=True visits t = L-1 .. 0.  zoh=True writes with the zero-order-hold
    coefficient (exp(dt A) - 1) / A instead of dt (every scan entry point
    takes delta_softplus and zoh).  conv_w [dim, 4] (and conv_b [dim]): u is
    the content before the block's causal conv and the scan runs on
    SiLU(conv(u)) computed in the kernel (vm_scan_dir.conv_w; direction dicts
    of vm_bidir_scan_fwd take the same keys)."""
    dt = u.dtype
    batch, dim, L = u.shape
    N = A.shape[-1]
    d, keep = _direction(dict(u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias,
                              conv_w=conv_w, conv_b=conv_b),
                         batch, dim, (batch, dim, L), L, N, dt, u.device, "p")
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    out = torch.empty_like(u) if out is None else _dev(out, "out", dt, u.shape, u.device)
    with torch.cuda.device(u.device):
        st = load_library().vm_selective_scan_fwd(ctypes.byref(d), _ptr(z), _ptr(out), batch, dim, L, N,
                                                  _dtype_code(u), _options(delta_softplus, zoh),
                                                  int(bool(reverse)), _stream(u.device))
    _check(st, "vm_selective_scan_fwd")
    return out


def vm_bidir_scan_fwd(fwd, bwd, z=None, combine_scale=1.0, delta_softplus=True, out=None, zoh=False):
    """Bidirectional scan: combine_scale * (y_fwd + y_bwd) * SiLU(z).
    fwd / bwd: dicts with u, delta, A, B, C, D, delta_bias (original token order)."""
    u = fwd["u"]
    dt = u.dtype
    batch, dim, L = u.shape
    N = fwd["A"].shape[-1]
    df, kf = _direction(fwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "fwd")
    db, kb = _direction(bwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "bwd")
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    out = torch.empty_like(u) if out is None else _dev(out, "out", dt, u.shape, u.device)
    with torch.cuda.device(u.device):
        st = load_library().vm_bidir_scan_fwd(ctypes.byref(df), ctypes.byref(db), _ptr(z),
                                              float(combine_scale), _ptr(out), batch, dim, L, N,
                                              _dtype_code(u), _options(delta_softplus, zoh),
                                              _stream(u.device))
    _check(st, "vm_bidir_scan_fwd")
    return out


def vm_bidir_scan_fwd_noalloc(fwd, bwd, out, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """vm_bidir_scan_fwd for callers that cannot allocate device memory: the
    same result, written into the caller's `out`; the exchange buffer of long
    sequences comes from a library-owned device array (batch * dim * (L
    rounded up to 32) <= 8388608, else VmError).  Calls on one GPU share that
    array: calls that overlap in time on one GPU must not be issued."""
    u = fwd["u"]
    dt = u.dtype
    batch, dim, L = u.shape
    N = fwd["A"].shape[-1]
    df, kf = _direction(fwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "fwd")
    db, kb = _direction(bwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "bwd")
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    _dev(out, "out", dt, u.shape, u.device)
    with torch.cuda.device(u.device):
        st = load_library().vm_bidir_scan_fwd_noalloc(ctypes.byref(df), ctypes.byref(db), _ptr(z),
                                                      float(combine_scale), _ptr(out), batch, dim, L, N,
                                                      _dtype_code(u), _options(delta_softplus, zoh),
                                                      _stream(u.device))
    _check(st, "vm_bidir_scan_fwd_noalloc")
    return out


def vm_causal_conv1d_silu(x, w, bias=None, reverse=False, out=None):
    """u = SiLU(depthwise causal conv of width 4 (+ bias)) per row of
    x [batch, dim, L]; w [dim, 4] fp32 (w[:, 3] on the current token);
    reverse=True convolves in reversed order (the backward branch)."""
    _dev(x, "x")
    dim = x.shape[1]
    _dev(w, "w", torch.float32, (dim, 4), x.device)
    if bias is not None:
        _dev(bias, "bias", torch.float32, (dim,), x.device)
    out = torch.empty_like(x) if out is None else _dev(out, "out", x.dtype, x.shape, x.device)
    batch, dim, L = x.shape
    with torch.cuda.device(x.device):
        st = load_library().vm_causal_conv1d_silu(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), batch, dim,
                                                  L, int(bool(reverse)), _dtype_code(x),
                                                  _stream(x.device))
    _check(st, "vm_causal_conv1d_silu")
    return out


def vm_causal_conv1d_silu_bwd(x, w, du, bias=None, reverse=False, with_dbias=None):
    """Gradients of sum(du * vm_causal_conv1d_silu(x, w, bias, reverse)):
    returns (dx, dw, dbias), fp32; du fp32 [batch, dim, L].  dbias is None
    when with_dbias is false (default: computed when bias is given)."""
    _dev(x, "x")
    batch, dim, L = x.shape
    _dev(w, "w", torch.float32, (dim, 4), x.device)
    _dev(du, "du", torch.float32, x.shape, x.device)
    if bias is not None:
        _dev(bias, "bias", torch.float32, (dim,), x.device)
    if with_dbias is None:
        with_dbias = bias is not None
    dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    dw = torch.empty((dim, 4), dtype=torch.float32, device=x.device)
    db = torch.empty((dim,), dtype=torch.float32, device=x.device) if with_dbias else None
    with torch.cuda.device(x.device):
        st = load_library().vm_causal_conv1d_silu_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(du), _ptr(dx),
                                                      _ptr(dw), _ptr(db), batch, dim, L,
                                                      int(bool(reverse)), _dtype_code(x), _stream(x.device))
    _check(st, "vm_causal_conv1d_silu_bwd")
    return dx, dw, db


def _grad_set(p, batch, dim, L, N, device, with_bias):
    """Gradient buffers of one direction; with the fused conv (p["conv_w"])
    also conv_w (and conv_b when p has one), and u is then the conv input's."""
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=device)
    conv = p.get("conv_w") is not None
    g = dict(u=f(batch, dim, L), delta=f(batch, dim, L), A=f(dim, N), B=f(batch, N, L),
             C=f(batch, N, L), D=f(dim), delta_bias=f(dim) if with_bias else None)
    if conv:
        g["conv_w"] = f(dim, 4)
        g["conv_b"] = f(dim) if p.get("conv_b") is not None else None
    ptr = lambda k: g[k].data_ptr() if g.get(k) is not None else None
    s = VmScanGrad(*(ptr(k) for k in ("u", "delta", "A", "B", "C", "D", "delta_bias", "conv_w", "conv_b")))
    return s, g


def vm_selective_scan_bwd(p, dout, z=None, delta_softplus=True, reverse=False, zoh=False):
    """Gradients of sum(dout * vm_selective_scan_fwd(**p, z=z, ...)).  p: dict
    u, delta, A, B, C, D, delta_bias (token tensors fp32 or bf16, like dout and
    z).  Returns (grads, dz), fp32: grads has the keys of p (dB, dC dense
    [batch, N, L]); dz is None without z."""
    u = p["u"]
    dt = u.dtype
    batch, dim, L = u.shape
    N = p["A"].shape[-1]
    d, keep = _direction(p, batch, dim, (batch, dim, L), L, N, dt, u.device, "p")
    _dev(dout, "dout", dt, u.shape, u.device)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    gs, g = _grad_set(p, batch, dim, L, N, u.device, p.get("delta_bias") is not None)
    dz = torch.empty(u.shape, dtype=torch.float32, device=u.device) if z is not None else None
    with torch.cuda.device(u.device):
        st = load_library().vm_selective_scan_bwd(ctypes.byref(d), _ptr(z), _ptr(dout), ctypes.byref(gs),
                                                  _ptr(dz), batch, dim, L, N, _dtype_code(u),
                                                  _options(delta_softplus, zoh), int(bool(reverse)),
                                                  _stream(u.device))
    _check(st, "vm_selective_scan_bwd")
    return g, dz


def vm_bidir_scan_bwd(fwd, bwd, dout, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Gradients of sum(dout * vm_bidir_scan_fwd(fwd, bwd, z, combine_scale)).
    Returns (grads of fwd, grads of bwd, dz), fp32 for fp32 or bf16 inputs."""
    u = fwd["u"]
    dt = u.dtype
    batch, dim, L = u.shape
    N = fwd["A"].shape[-1]
    df, kf = _direction(fwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "fwd")
    db, kb = _direction(bwd, batch, dim, (batch, dim, L), L, N, dt, u.device, "bwd")
    _dev(dout, "dout", dt, u.shape, u.device)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    gsf, gf = _grad_set(fwd, batch, dim, L, N, u.device, fwd.get("delta_bias") is not None)
    gsb, gb = _grad_set(bwd, batch, dim, L, N, u.device, bwd.get("delta_bias") is not None)
    dz = torch.empty(u.shape, dtype=torch.float32, device=u.device) if z is not None else None
    with torch.cuda.device(u.device):
        st = load_library().vm_bidir_scan_bwd(ctypes.byref(df), ctypes.byref(db), _ptr(z), _ptr(dout),
                                              float(combine_scale), ctypes.byref(gsf), ctypes.byref(gsb),
                                              _ptr(dz), batch, dim, L, N, _dtype_code(u),
                                              _options(delta_softplus, zoh), _stream(u.device))
    _check(st, "vm_bidir_scan_bwd")
    return gf, gb, dz


def vm_atrous_group_len(height: int, width: int) -> int:
    n = int(load_library().vm_atrous_group_len(int(height), int(width)))
    if n < 0:
        raise VmError(-n, f"vm_atrous_group_len: {vm_status_string(-n)}")
    return n


def vm_atrous_gather(x, out=None):
    """x [batch, ch, H, W] -> streams [batch, 4, ch, ceil(H/2)*ceil(W/2)]."""
    _dev(x, "x")
    batch, ch, H, W = x.shape
    shape = (batch, 4, ch, vm_atrous_group_len(H, W))
    out = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else \
        _dev(out, "streams", x.dtype, shape, x.device)
    with torch.cuda.device(x.device):
        st = load_library().vm_atrous_gather(_ptr(x), _ptr(out), batch, ch, H, W, _dtype_code(x),
                                             _stream(x.device))
    _check(st, "vm_atrous_gather")
    return out


def vm_atrous_scatter(streams, height, width, out=None):
    """streams [batch, 4, ch, Lg] -> y [batch, ch, height, width]."""
    _dev(streams, "streams")
    batch, four, ch, Lg = streams.shape
    if four != 4 or Lg != vm_atrous_group_len(height, width):
        raise ValueError("streams must be [batch, 4, ch, ceil(H/2)*ceil(W/2)]")
    shape = (batch, ch, height, width)
    out = torch.empty(shape, dtype=streams.dtype, device=streams.device) if out is None else \
        _dev(out, "y", streams.dtype, shape, streams.device)
    with torch.cuda.device(streams.device):
        st = load_library().vm_atrous_scatter(_ptr(streams), _ptr(out), batch, ch, height, width,
                                              _dtype_code(streams), _stream(streams.device))
    _check(st, "vm_atrous_scatter")
    return out


def vm_pool_scan_repeat(fwd, bwd=None, z=None, combine_scale=1.0, pool_axis=0, delta_softplus=True,
                        out=None, zoh=False):
    """FastVim pooled scan.  Per direction: u [batch, dim, H, W], delta
    [batch, dim, Lp], B/C [batch, N, Lp] (Lp = H for pool_axis 0, W for 1).
    Returns [batch, dim, H, W]."""
    u = fwd["u"]
    dt = u.dtype
    batch, dim, H, W = u.shape
    Lp = H if pool_axis == 0 else W
    N = fwd["A"].shape[-1]
    df, kf = _direction(fwd, batch, dim, (batch, dim, H, W), Lp, N, dt, u.device, "fwd")
    pb = None
    if bwd is not None:
        db, kb = _direction(bwd, batch, dim, (batch, dim, H, W), Lp, N, dt, u.device, "bwd")
        pb = ctypes.byref(db)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    out = torch.empty_like(u) if out is None else _dev(out, "out", dt, u.shape, u.device)
    with torch.cuda.device(u.device):
        st = load_library().vm_pool_scan_repeat(ctypes.byref(df), pb, _ptr(z), float(combine_scale),
                                                _ptr(out), batch, dim, H, W, N, int(pool_axis),
                                                _dtype_code(u), _options(delta_softplus, zoh),
                                                _stream(u.device))
    _check(st, "vm_pool_scan_repeat")
    return out


def vm_pool_scan_repeat_bwd(fwd, dout, bwd=None, z=None, combine_scale=1.0, pool_axis=0,
                            delta_softplus=True, zoh=False):
    """Gradients of sum(dout * vm_pool_scan_repeat(fwd, bwd, z, ...)).
    Returns (grads of fwd, grads of bwd or None, dz or None), fp32: u's
    gradient at full resolution, the others at the pooled length."""
    u = fwd["u"]
    dt = u.dtype
    batch, dim, H, W = u.shape
    Lp = H if pool_axis == 0 else W
    N = fwd["A"].shape[-1]
    df, kf = _direction(fwd, batch, dim, (batch, dim, H, W), Lp, N, dt, u.device, "fwd")
    pb, gsb, gb = None, None, None
    if bwd is not None:
        db, kb = _direction(bwd, batch, dim, (batch, dim, H, W), Lp, N, dt, u.device, "bwd")
        pb = ctypes.byref(db)
    _dev(dout, "dout", dt, u.shape, u.device)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)

    def grad_set(p):
        s_, g_ = _grad_set(p, batch, dim, Lp, N, u.device, p.get("delta_bias") is not None)
        g_["u"] = torch.empty(u.shape, dtype=torch.float32, device=u.device)   # full resolution
        s_.du = g_["u"].data_ptr()
        return s_, g_

    gsf, gf = grad_set(fwd)
    if bwd is not None:
        gsb, gb = grad_set(bwd)
    dz = torch.empty(u.shape, dtype=torch.float32, device=u.device) if z is not None else None
    with torch.cuda.device(u.device):
        st = load_library().vm_pool_scan_repeat_bwd(
            ctypes.byref(df), pb, _ptr(z), _ptr(dout), float(combine_scale), ctypes.byref(gsf),
            ctypes.byref(gsb) if gsb is not None else None, _ptr(dz), batch, dim, H, W, N,
            int(pool_axis), _dtype_code(u), _options(delta_softplus, zoh), _stream(u.device))
    _check(st, "vm_pool_scan_repeat_bwd")
    return gf, gb, dz


def vm_ss2d_scan_fwd(u, dirs, z=None, combine_scale=1.0, delta_softplus=True, out=None, zoh=False):
    """Four-direction 2-D scan with summed merge.  u, z: [batch, dim, H, W].
    dirs: four dicts with delta, A, B, C, D, delta_bias (a "u" key is
    ignored); traversals 0 / 1 are row-major forward / reversed, 2 / 3
    column-major forward / reversed, and each indexes its delta [batch, dim,
    H*W] and B, C [batch, N, H*W] by its own traversal step.
    Returns combine_scale * (sum of the four aligned outputs) * SiLU(z)."""
    _dev(u, "u")
    dt = u.dtype
    batch, dim, H, W = u.shape
    if len(dirs) != 4:
        raise ValueError("dirs must hold four traversals")
    N = dirs[0]["A"].shape[-1]
    arr = (VmScanDir * 4)()
    keep = []
    for k, p in enumerate(dirs):
        d, kp = _direction(dict(p, u=u), batch, dim, (batch, dim, H, W), H * W, N, dt, u.device,
                           f"dirs[{k}]")
        arr[k] = d
        keep.append(kp)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    out = torch.empty_like(u) if out is None else _dev(out, "out", dt, u.shape, u.device)
    with torch.cuda.device(u.device):
        st = load_library().vm_ss2d_scan_fwd(arr, _ptr(u), _ptr(z), float(combine_scale), _ptr(out),
                                             batch, dim, H, W, N, _dtype_code(u),
                                             _options(delta_softplus, zoh), _stream(u.device))
    _check(st, "vm_ss2d_scan_fwd")
    return out


def vm_ss2d_scan_bwd(u, dirs, dout, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Gradients of sum(dout * vm_ss2d_scan_fwd(u, dirs, z, combine_scale)).
    Returns (du [batch, dim, H, W], per-traversal grads (four dicts with the
    keys of dirs, dB / dC dense [batch, N, H*W]), dz or None), all fp32."""
    _dev(u, "u")
    dt = u.dtype
    batch, dim, H, W = u.shape
    if len(dirs) != 4:
        raise ValueError("dirs must hold four traversals")
    N = dirs[0]["A"].shape[-1]
    arr = (VmScanDir * 4)()
    garr = (VmScanGrad * 4)()
    keep, grads = [], []
    for k, p in enumerate(dirs):
        d, kp = _direction(dict(p, u=u), batch, dim, (batch, dim, H, W), H * W, N, dt, u.device,
                           f"dirs[{k}]")
        arr[k] = d
        keep.append(kp)
        gs, g = _grad_set(dict(p, u=u), batch, dim, H * W, N, u.device, p.get("delta_bias") is not None)
        del g["u"]                  # the map's gradient is the summed du below
        gs.du = None
        garr[k] = gs
        grads.append(g)
    _dev(dout, "dout", dt, u.shape, u.device)
    if z is not None:
        _dev(z, "z", dt, u.shape, u.device)
    du = torch.empty(u.shape, dtype=torch.float32, device=u.device)
    dz = torch.empty(u.shape, dtype=torch.float32, device=u.device) if z is not None else None
    with torch.cuda.device(u.device):
        st = load_library().vm_ss2d_scan_bwd(arr, _ptr(u), _ptr(z), _ptr(dout), float(combine_scale), garr,
                                             _ptr(du), _ptr(dz), batch, dim, H, W, N, _dtype_code(u),
                                             _options(delta_softplus, zoh), _stream(u.device))
    _check(st, "vm_ss2d_scan_bwd")
    return du, grads, dz


__all__ = ["vm_selective_scan_fwd", "vm_bidir_scan_fwd", "vm_bidir_scan_fwd_noalloc", "vm_atrous_gather", "vm_atrous_scatter",
           "vm_pool_scan_repeat", "vm_ss2d_scan_fwd", "vm_causal_conv1d_silu",
           "vm_causal_conv1d_silu_bwd", "vm_pool_scan_repeat_bwd", "vm_ss2d_scan_bwd",
           "vm_selective_scan_bwd", "vm_bidir_scan_bwd", "VmScanGrad", "vm_atrous_group_len", "vm_status_string", "vm_version",
           "VmScanDir", "VmError", "load_library", "LIB_PATH", "EXPORTED"]
