"""Pins for the gradient oracle (no GPU): its forward equals the C oracle's,
and every gradient it returns equals a central finite difference of the C
oracle's forward (an independent implementation)."""
import importlib.util
import os

import numpy as np
import pytest

import oracle


def _grad_oracle():
    """The gradient oracle; VM_GRAD_ORACLE names a deliberately broken copy
    of it (tests/test_oracle_grad_mutants.py), never set in normal runs."""
    path = os.environ.get("VM_GRAD_ORACLE")
    if not path:
        from oracle import grad
        return grad
    spec = importlib.util.spec_from_file_location("grad_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


og = _grad_oracle()


def _rng(seed):
    return np.random.default_rng(seed)


def _dir(rng, batch, dim, L, N):
    return dict(u=rng.standard_normal((batch, dim, L)),
                delta=rng.standard_normal((batch, dim, L)) * 0.5,
                A=-rng.uniform(0.2, 2.0, size=(dim, N)),
                B=rng.standard_normal((batch, N, L)),
                C=rng.standard_normal((batch, N, L)),
                D=rng.standard_normal(dim),
                delta_bias=rng.uniform(-1.0, 0.5, size=dim))


def _fd(f, p, key, eps=1e-6):
    """Central differences of the scalar f(p) with respect to p[key]."""
    base = p[key]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        hi, lo = base.copy(), base.copy()
        hi[i] += eps
        lo[i] -= eps
        g[i] = (f(dict(p, **{key: hi})) - f(dict(p, **{key: lo}))) / (2 * eps)
    return g


def _check(got, want, what):
    scale = max(1.0, float(np.max(np.abs(want))))
    err = float(np.max(np.abs(got - want)))
    assert err <= 2e-7 * scale, f"{what}: max abs error {err:.3e} (scale {scale:.2e})"


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("softplus", [True, False])
def test_single_grad_matches_finite_differences(reverse, gated, softplus):
    rng = _rng(80 + 4 * reverse + 2 * gated + softplus)
    p = _dir(rng, 2, 2, 5, 3)
    if not softplus:
        p["delta"] = rng.uniform(0.05, 0.6, size=p["delta"].shape)
    z = rng.standard_normal(p["u"].shape) if gated else None
    dout = rng.standard_normal(p["u"].shape)
    g, dz, out = og.selective_scan_grad(p, dout, z=z, delta_softplus=softplus, reverse=reverse)
    f = lambda q, zz=z: float(np.sum(dout * oracle.selective_scan(**q, z=zz, delta_softplus=softplus,
                                                                   reverse=reverse)))
    np.testing.assert_allclose(out, oracle.selective_scan(**p, z=z, delta_softplus=softplus,
                                                          reverse=reverse), rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(g[k], _fd(f, p, k), k)
    if gated:
        _check(dz, _fd(lambda q: f(p, q["z"]), dict(z=z), "z"), "z")


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("gated", [False, True])
def test_zoh_grad_matches_finite_differences(reverse, gated):
    """The zero-order-hold write: one column of A is 0 (coefficient dt, whose
    A-derivative dt^2 / 2 the series keeps), others span small and large
    |dt A| on both sides of the oracle's series switch."""
    rng = _rng(110 + 2 * reverse + gated)
    p = _dir(rng, 2, 2, 5, 4)
    p["A"][:, 0] = 0.0
    p["A"][0, 1] = -1e-4
    z = rng.standard_normal(p["u"].shape) if gated else None
    dout = rng.standard_normal(p["u"].shape)
    g, dz, out = og.selective_scan_grad(p, dout, z=z, reverse=reverse, zoh=True)
    f = lambda q, zz=z: float(np.sum(dout * oracle.selective_scan(**q, z=zz, reverse=reverse, zoh=True)))
    np.testing.assert_allclose(out, oracle.selective_scan(**p, z=z, reverse=reverse, zoh=True),
                               rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(g[k], _fd(f, p, k), k)
    if gated:
        _check(dz, _fd(lambda q: f(p, q["z"]), dict(z=z), "z"), "z")


def test_zoh_bidir_grad_matches_finite_differences():
    rng = _rng(120)
    f_, b_ = _dir(rng, 1, 2, 6, 3), _dir(rng, 1, 2, 6, 3)
    z = rng.standard_normal(f_["u"].shape)
    dout = rng.standard_normal(f_["u"].shape)
    gf, gb, dz, out = og.bidir_scan_grad(f_, b_, dout, z=z, combine_scale=0.5, zoh=True)
    fn = lambda ff, bb, zz=z: float(np.sum(dout * oracle.bidir_scan(ff, bb, z=zz, combine_scale=0.5,
                                                                     zoh=True)))
    np.testing.assert_allclose(out, oracle.bidir_scan(f_, b_, z=z, combine_scale=0.5, zoh=True),
                               rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(gf[k], _fd(lambda q: fn(q, b_), f_, k), "fwd " + k)
        _check(gb[k], _fd(lambda q: fn(f_, q), b_, k), "bwd " + k)
    _check(dz, _fd(lambda q: fn(f_, b_, q["z"]), dict(z=z), "z"), "z")


def test_zoh_grad_differs_from_released_write():
    """Guard against the flag being ignored: on steps with |dt A| near 1 the
    two discretisations' gradients differ well beyond the tolerance."""
    rng = _rng(130)
    p = _dir(rng, 1, 2, 4, 2)
    dout = rng.standard_normal(p["u"].shape)
    g0, _, _ = og.selective_scan_grad(p, dout)
    g1, _, _ = og.selective_scan_grad(p, dout, zoh=True)
    for k in ("u", "delta", "A", "B"):
        assert np.max(np.abs(g0[k] - g1[k])) > 1e-3, k


def test_bidir_grad_matches_finite_differences():
    rng = _rng(90)
    f_, b_ = _dir(rng, 1, 2, 6, 3), _dir(rng, 1, 2, 6, 3)
    z = rng.standard_normal(f_["u"].shape)
    dout = rng.standard_normal(f_["u"].shape)
    gf, gb, dz, out = og.bidir_scan_grad(f_, b_, dout, z=z, combine_scale=0.5)
    fn = lambda ff, bb, zz=z: float(np.sum(dout * oracle.bidir_scan(ff, bb, z=zz, combine_scale=0.5)))
    np.testing.assert_allclose(out, oracle.bidir_scan(f_, b_, z=z, combine_scale=0.5), rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(gf[k], _fd(lambda q: fn(q, b_), f_, k), "fwd " + k)
        _check(gb[k], _fd(lambda q: fn(f_, q), b_, k), "bwd " + k)
    _check(dz, _fd(lambda q: fn(f_, b_, q["z"]), dict(z=z), "z"), "z")


def test_grad_of_skip_only_case():
    # B = 0: the state stays 0, y = D u; so du = D * dout, dD = sum(dout * u),
    # and nothing reaches delta, A, C (closed form, no finite differences)
    rng = _rng(91)
    p = _dir(rng, 2, 3, 4, 2)
    p["B"] = np.zeros_like(p["B"])
    dout = rng.standard_normal(p["u"].shape)
    g, _, _ = og.selective_scan_grad(p, dout)
    np.testing.assert_allclose(g["u"], p["D"][None, :, None] * dout, rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["D"], (dout * p["u"]).sum(axis=(0, 2)), rtol=0, atol=1e-13)
    for k in ("delta", "A", "C", "delta_bias"):
        assert np.all(g[k] == 0.0), k


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("L", [1, 2, 7])
def test_conv_grad_matches_finite_differences(reverse, L):
    """Conv + SiLU gradients: rows shorter than the filter (L = 1, 2) keep
    only the taps inside the row."""
    rng = _rng(140 + 3 * L + reverse)
    p = dict(x=rng.standard_normal((2, 3, L)), w=rng.standard_normal((3, 4)) * 0.5,
             bias=rng.standard_normal(3) * 0.3)
    du = rng.standard_normal((2, 3, L))
    dx, dw, db, u = og.causal_conv1d_silu_grad(p["x"], p["w"], p["bias"], du, reverse=reverse)
    np.testing.assert_allclose(u, oracle.causal_conv1d_silu(p["x"], p["w"], p["bias"], reverse=reverse),
                               rtol=0, atol=1e-13)
    f = lambda q: float(np.sum(du * oracle.causal_conv1d_silu(q["x"], q["w"], q["bias"], reverse=reverse)))
    _check(dx, _fd(f, p, "x"), "x")
    _check(dw, _fd(f, p, "w"), "w")
    _check(db, _fd(f, p, "bias"), "bias")


def test_conv_grad_without_bias_and_tap_structure():
    """No bias: dbias is None.  Brute force on one row: dx[s] collects
    w[k] dv[s + 3 - k] from the outputs that read x[s]."""
    rng = _rng(150)
    x = rng.standard_normal((1, 1, 6))
    w = rng.standard_normal((1, 4))
    du = rng.standard_normal((1, 1, 6))
    dx, dw, db, _ = og.causal_conv1d_silu_grad(x, w, None, du)
    assert db is None
    v = np.array([sum(w[0, k] * x[0, 0, t - 3 + k] for k in range(4) if t - 3 + k >= 0) for t in range(6)])
    s = 1 / (1 + np.exp(-v))
    dv = du[0, 0] * s * (1 + v * (1 - s))
    want = np.array([sum(w[0, k] * dv[s_ + 3 - k] for k in range(4) if 0 <= s_ + 3 - k < 6)
                     for s_ in range(6)])
    np.testing.assert_allclose(dx[0, 0], want, rtol=1e-12, atol=1e-12)
    want_w = np.array([sum(dv[t] * x[0, 0, t - 3 + k] for t in range(6) if t - 3 + k >= 0)
                       for k in range(4)])
    np.testing.assert_allclose(dw[0], want_w, rtol=1e-12, atol=1e-12)


def _pool_dir(rng, batch, dim, H, W, Lp, N):
    return dict(u=rng.standard_normal((batch, dim, H, W)),
                delta=rng.standard_normal((batch, dim, Lp)) * 0.5,
                A=-rng.uniform(0.2, 2.0, size=(dim, N)),
                B=rng.standard_normal((batch, N, Lp)),
                C=rng.standard_normal((batch, N, Lp)),
                D=rng.standard_normal(dim),
                delta_bias=rng.uniform(-1.0, 0.5, size=dim))


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("bidir", [False, True])
def test_pool_grad_matches_finite_differences(axis, bidir):
    rng = _rng(160 + 2 * axis + bidir)
    H, W = 3, 4
    Lp = H if axis == 0 else W
    f_ = _pool_dir(rng, 1, 2, H, W, Lp, 3)
    b_ = _pool_dir(rng, 1, 2, H, W, Lp, 3) if bidir else None
    z = rng.standard_normal(f_["u"].shape)
    dout = rng.standard_normal(f_["u"].shape)
    gf, gb, dz, out = og.pool_scan_repeat_grad(f_, b_, dout, z=z, combine_scale=0.5, pool_axis=axis)
    fn = lambda ff, bb, zz=z: float(np.sum(dout * oracle.pool_scan_repeat(ff, bb, z=zz, combine_scale=0.5,
                                                                           pool_axis=axis)))
    np.testing.assert_allclose(out, oracle.pool_scan_repeat(f_, b_, z=z, combine_scale=0.5, pool_axis=axis),
                               rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(gf[k], _fd(lambda q: fn(q, b_), f_, k), "fwd " + k)
        if bidir:
            _check(gb[k], _fd(lambda q: fn(f_, q), b_, k), "bwd " + k)
    _check(dz, _fd(lambda q: fn(f_, b_, q["z"]), dict(z=z), "z"), "z")


@pytest.mark.parametrize("H,W", [(2, 3), (3, 2)])
def test_ss2d_grad_matches_finite_differences(H, W):
    rng = _rng(170 + H)
    L = H * W
    u = rng.standard_normal((1, 2, H, W))
    dirs = []
    for _ in range(4):
        d = _dir(rng, 1, 2, L, 3)
        d.pop("u")
        dirs.append(d)
    z = rng.standard_normal(u.shape)
    dout = rng.standard_normal(u.shape)
    du, gd, dz, out = og.ss2d_scan_grad(u, dirs, dout, z=z, combine_scale=0.5)
    fn = lambda uu, dd, zz=z: float(np.sum(dout * oracle.ss2d_scan(uu, dd, z=zz, combine_scale=0.5)))
    np.testing.assert_allclose(out, oracle.ss2d_scan(u, dirs, z=z, combine_scale=0.5), rtol=0, atol=1e-12)
    _check(du, _fd(lambda q: fn(q["u"], dirs), dict(u=u), "u"), "u")
    for k in range(4):
        for key in ("delta", "A", "B", "C", "D", "delta_bias"):
            f = lambda q, k=k: fn(u, [q if j == k else dirs[j] for j in range(4)])
            _check(gd[k][key], _fd(f, dirs[k], key), f"dir{k} {key}")
    _check(dz, _fd(lambda q: fn(u, dirs, q["z"]), dict(z=z), "z"), "z")



def _zoh_A(A):
    """One A column at 0 (coefficient dt; the series' A-derivative dt^2 / 2)
    and one entry small enough to take the oracle's series branch."""
    A = A.copy()
    A[:, 0] = 0.0
    A[0, 1] = -1e-4
    return A


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("bidir", [False, True])
def test_zoh_pool_grad_matches_finite_differences(axis, bidir):
    """The pooled path with the zero-order-hold write ("Norm or Direction?"
    page, section 3, eq. 2; FastVim summary, "Methodology": A and B
    discretised by zero-order hold), on both pooling axes, with and without
    the backward direction."""
    rng = _rng(180 + 2 * axis + bidir)
    H, W = 3, 4
    Lp = H if axis == 0 else W
    f_ = _pool_dir(rng, 1, 2, H, W, Lp, 3)
    f_["A"] = _zoh_A(f_["A"])
    b_ = _pool_dir(rng, 1, 2, H, W, Lp, 3) if bidir else None
    if bidir:
        b_["A"] = _zoh_A(b_["A"])
    z = rng.standard_normal(f_["u"].shape)
    dout = rng.standard_normal(f_["u"].shape)
    gf, gb, dz, out = og.pool_scan_repeat_grad(f_, b_, dout, z=z, combine_scale=0.5, pool_axis=axis,
                                               zoh=True)
    fn = lambda ff, bb, zz=z: float(np.sum(dout * oracle.pool_scan_repeat(
        ff, bb, z=zz, combine_scale=0.5, pool_axis=axis, zoh=True)))
    np.testing.assert_allclose(out, oracle.pool_scan_repeat(f_, b_, z=z, combine_scale=0.5, pool_axis=axis,
                                                            zoh=True), rtol=0, atol=1e-12)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        _check(gf[k], _fd(lambda q: fn(q, b_), f_, k), "fwd " + k)
        if bidir:
            _check(gb[k], _fd(lambda q: fn(f_, q), b_, k), "bwd " + k)
    _check(dz, _fd(lambda q: fn(f_, b_, q["z"]), dict(z=z), "z"), "z")


def test_zoh_ss2d_grad_matches_finite_differences():
    """SS2D with the zero-order-hold write ("Norm or Direction?" page, section
    3, eq. 2 and "2D Selective Scan (SS2D)"): every traversal's gradients."""
    rng = _rng(190)
    H, W = 2, 3
    L = H * W
    u = rng.standard_normal((1, 2, H, W))
    dirs = []
    for _ in range(4):
        d = _dir(rng, 1, 2, L, 3)
        d.pop("u")
        d["A"] = _zoh_A(d["A"])
        dirs.append(d)
    z = rng.standard_normal(u.shape)
    dout = rng.standard_normal(u.shape)
    du, gd, dz, out = og.ss2d_scan_grad(u, dirs, dout, z=z, combine_scale=0.5, zoh=True)
    fn = lambda uu, dd, zz=z: float(np.sum(dout * oracle.ss2d_scan(uu, dd, z=zz, combine_scale=0.5, zoh=True)))
    np.testing.assert_allclose(out, oracle.ss2d_scan(u, dirs, z=z, combine_scale=0.5, zoh=True),
                               rtol=0, atol=1e-12)
    _check(du, _fd(lambda q: fn(q["u"], dirs), dict(u=u), "u"), "u")
    for k in range(4):
        for key in ("delta", "A", "B", "C", "D", "delta_bias"):
            f = lambda q, k=k: fn(u, [q if j == k else dirs[j] for j in range(4)])
            _check(gd[k][key], _fd(f, dirs[k], key), f"dir{k} {key}")
    _check(dz, _fd(lambda q: fn(u, dirs, q["z"]), dict(z=z), "z"), "z")
