"""fp64 CPU oracle for the selective-scan hot path (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its Python
binding) never imports, links or calls it.  The arithmetic lives in plain C
(``vm_oracle.c``); this module only converts numpy arrays to float64, calls
the C functions through ctypes and returns numpy arrays.  Each wrapper names
the page passage its C function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vm_oracle.c")
# VM_ORACLE_LIB lets the test suite load a deliberately broken build of this
# oracle (see tests/test_oracle_mutants.py); normal runs never set it.
_LIB_PATH = os.environ.get("VM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile vm_oracle.c with gcc into liboracle.so (OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.vmo_num_threads.restype = ctypes.c_int
            lib.vmo_selective_scan.argtypes = [_D] * 8 + [_I64] * 4 + [ctypes.c_int] * 3 + [_D]
            lib.vmo_bidir_scan.argtypes = ([_D] * 15 + [ctypes.c_double] + [_I64] * 4
                                           + [ctypes.c_int] * 2 + [_D])
            lib.vmo_atrous_group_len.argtypes = [_I64, _I64]
            lib.vmo_atrous_group_len.restype = _I64
            lib.vmo_atrous_route.argtypes = [_I64, _I64, ctypes.c_int,
                                             ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
            lib.vmo_atrous_gather.argtypes = [_D] + [_I64] * 4 + [_D]
            lib.vmo_atrous_scatter.argtypes = [_D] + [_I64] * 4 + [_D]
            lib.vmo_mean_pool.argtypes = [_D] + [_I64] * 4 + [ctypes.c_int, _D]
            lib.vmo_pool_scan_repeat.argtypes = ([_D] * 15 + [ctypes.c_double] + [_I64] * 5
                                                 + [ctypes.c_int] * 3 + [_D])
            _D4 = _D * 4
            lib.vmo_ss2d_scan.argtypes = ([_D] + [_D4] * 6 + [_D, ctypes.c_double] + [_I64] * 5
                                          + [ctypes.c_int] * 2 + [_D])
            lib.vmo_causal_conv1d_silu.argtypes = [_D] * 3 + [_I64] * 3 + [ctypes.c_int, _D]
            for name in ("vmo_selective_scan", "vmo_bidir_scan", "vmo_atrous_route",
                         "vmo_atrous_gather", "vmo_atrous_scatter", "vmo_mean_pool",
                         "vmo_pool_scan_repeat", "vmo_ss2d_scan", "vmo_causal_conv1d_silu"):
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's row loop uses."""
    return int(_load().vmo_num_threads())


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _check(status, what):
    if status != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {status})")


def selective_scan(u, delta, A, B, C, D, z=None, delta_bias=None,
                   delta_softplus=True, reverse=False, zoh=False):
    """One-direction scan (Vim page, implementation row 4; reverse = the
    backward direction of "Two scans meet at the same token", done literally
    as flip, scan, flip).  u, delta, z: [batch, dim, L]; A: [dim, N];
    B, C: [batch, N, L]; D, delta_bias: [dim].  zoh=True writes with the
    zero-order-hold coefficient expm1(dt A) / A instead of dt ("Norm or
    Direction?" page, section 3, eq. 2).  Returns float64 [batch, dim, L]."""
    u, delta, A, B, C, D, z, delta_bias = map(_f64, (u, delta, A, B, C, D, z, delta_bias))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N) and B.shape == (batch, N, L)
    assert C.shape == B.shape and D.shape == (dim,)
    assert z is None or z.shape == u.shape
    assert delta_bias is None or delta_bias.shape == (dim,)
    out = np.empty_like(u)
    _check(_load().vmo_selective_scan(_p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
                                      _p(delta_bias), batch, dim, L, N, int(bool(delta_softplus)),
                                      int(bool(zoh)), int(bool(reverse)), _p(out)), "selective_scan")
    return out


def causal_conv1d_silu(x, w, bias=None, reverse=False):
    """Depthwise causal conv of width 4 plus bias, then SiLU (Vim page,
    "Inside the released Vim block"); reverse=True is the backward branch's
    (flip, convolve, flip back).  x: [batch, dim, L]; w: [dim, 4] (w[:, 3] on
    the current token); bias: [dim].  Returns float64 [batch, dim, L]."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    batch, dim, L = x.shape
    assert w.shape == (dim, 4) and (bias is None or bias.shape == (dim,))
    out = np.empty_like(x)
    _check(_load().vmo_causal_conv1d_silu(_p(x), _p(w), _p(bias), batch, dim, L,
                                          int(bool(reverse)), _p(out)), "causal_conv1d_silu")
    return out


def _dir(p):
    """Unpack a direction dict {u, delta, A, B, C, D, delta_bias} to float64."""
    return [_f64(p.get(k)) for k in ("u", "delta", "A", "B", "C", "D", "delta_bias")]


def bidir_scan(fwd, bwd, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Bidirectional scan (Vim page, "Two scans meet at the same token" and
    implementation row 5): scale * (y_fwd + flip(scan(flip(bwd)))) * SiLU(z).
    fwd / bwd: dicts with u, delta, A, B, C, D, delta_bias (original order)."""
    uf, df, Af, Bf, Cf, Df, bf = _dir(fwd)
    ub, db, Ab, Bb, Cb, Db, bb = _dir(bwd)
    z = _f64(z)
    batch, dim, L = uf.shape
    N = Af.shape[1]
    for t in (uf, df, ub, db):
        assert t.shape == (batch, dim, L)
    out = np.empty_like(uf)
    _check(_load().vmo_bidir_scan(_p(uf), _p(df), _p(Af), _p(Bf), _p(Cf), _p(Df), _p(bf),
                                  _p(ub), _p(db), _p(Ab), _p(Bb), _p(Cb), _p(Db), _p(bb),
                                  _p(z), float(combine_scale), batch, dim, L, N,
                                  int(bool(delta_softplus)), int(bool(zoh)), _p(out)), "bidir_scan")
    return out


def atrous_group_len(H, W):
    """ceil(H/2) * ceil(W/2) (EfficientVMamba page, implementation row 1)."""
    n = int(_load().vmo_atrous_group_len(H, W))
    if n < 0:
        raise ValueError("non-positive spatial size")
    return n


def atrous_route(H, W, group):
    """(rows, cols) visited by the group's stream (EfficientVMamba page,
    "Four shorter sequences, one dense output"; padding coordinates included)."""
    n = atrous_group_len(H, W)
    rr = np.empty(n, dtype=np.int64)
    cc = np.empty(n, dtype=np.int64)
    _check(_load().vmo_atrous_route(H, W, group, rr.ctypes.data_as(ctypes.POINTER(_I64)),
                                    cc.ctypes.data_as(ctypes.POINTER(_I64))), "atrous_route")
    return rr, cc


def atrous_gather(x):
    """x [batch, ch, H, W] -> streams [batch, 4, ch, Lg], zero at padding."""
    x = _f64(x)
    batch, ch, H, W = x.shape
    out = np.empty((batch, 4, ch, atrous_group_len(H, W)), dtype=np.float64)
    _check(_load().vmo_atrous_gather(_p(x), batch, ch, H, W, _p(out)), "atrous_gather")
    return out


def atrous_scatter(streams, H, W):
    """streams [batch, 4, ch, Lg] -> y [batch, ch, H, W] (one owner per
    coordinate, padding cropped, nothing summed)."""
    s = _f64(streams)
    batch, four, ch, Lg = s.shape
    assert four == 4 and Lg == atrous_group_len(H, W)
    out = np.zeros((batch, ch, H, W), dtype=np.float64)
    _check(_load().vmo_atrous_scatter(_p(s), batch, ch, H, W, _p(out)), "atrous_scatter")
    return out


def mean_pool(u, axis):
    """[batch, dim, H, W] -> [batch, dim, Lp]; axis 0 averages over W, axis 1
    over H (FastVim summary, "Methodology")."""
    u = _f64(u)
    batch, dim, H, W = u.shape
    out = np.empty((batch, dim, H if axis == 0 else W), dtype=np.float64)
    _check(_load().vmo_mean_pool(_p(u), batch, dim, H, W, int(axis), _p(out)), "mean_pool")
    return out


def pool_scan_repeat(fwd, bwd, z=None, combine_scale=1.0, pool_axis=0, delta_softplus=True,
                     zoh=False):
    """FastVim pooled scan (FastVim summary, "Methodology"): pool u, scan the
    pooled sequence forward (and backward if bwd is given), repeat along the
    pooled axis, gate with SiLU(z) at full resolution.  fwd/bwd u are
    [batch, dim, H, W]; delta [batch, dim, Lp]; B, C [batch, N, Lp]."""
    uf, df, Af, Bf, Cf, Df, bf = _dir(fwd)
    if bwd is not None:
        ub, db, Ab, Bb, Cb, Db, bb = _dir(bwd)
    else:
        ub = db = Ab = Bb = Cb = Db = bb = None
    z = _f64(z)
    batch, dim, H, W = uf.shape
    N = Af.shape[1]
    out = np.empty_like(uf)
    _check(_load().vmo_pool_scan_repeat(_p(uf), _p(df), _p(Af), _p(Bf), _p(Cf), _p(Df), _p(bf),
                                        _p(ub), _p(db), _p(Ab), _p(Bb), _p(Cb), _p(Db), _p(bb),
                                        _p(z), float(combine_scale), batch, dim, H, W, N,
                                        int(pool_axis), int(bool(delta_softplus)), int(bool(zoh)),
                                        _p(out)),
           "pool_scan_repeat")
    return out


def ss2d_scan(u, dirs, z=None, combine_scale=1.0, delta_softplus=True, zoh=False):
    """Four-direction 2-D scan with summed merge ("Norm or Direction?" page,
    section 3, "2D Selective Scan (SS2D)"; EfficientVMamba page, "Merge
    restores coordinates instead of adding directions").  u, z: [batch, dim,
    H, W].  dirs: four dicts with delta, A, B, C, D, delta_bias; directions 0
    and 1 (row-major, then reversed) index delta, B, C by row-major step
    [batch, dim or N, H*W], directions 2 and 3 (column-major, then reversed)
    by column-major step.  Returns float64 [batch, dim, H, W]."""
    u, z = _f64(u), _f64(z)
    batch, dim, H, W = u.shape
    ds = [_dir(p) for p in dirs]
    assert len(ds) == 4
    N = ds[0][2].shape[1]
    for _, d, A, B, C, D, _b in ds:
        assert d.shape == (batch, dim, H * W) and A.shape == (dim, N)
        assert B.shape == (batch, N, H * W) and C.shape == B.shape and D.shape == (dim,)
    arr = lambda i: (_D * 4)(*[_p(x[i]) for x in ds])
    out = np.empty_like(u)
    _check(_load().vmo_ss2d_scan(_p(u), arr(1), arr(2), arr(3), arr(4), arr(5), arr(6), _p(z),
                                 float(combine_scale), batch, dim, H, W, N,
                                 int(bool(delta_softplus)), int(bool(zoh)), _p(out)), "ss2d_scan")
    return out
