"""Pins for the fp64 CPU oracle (no GPU needed).

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, a brute-force materialised-kernel sum written here
in plain Python, special cases with a textbook answer, and invariants.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_dir(rng, batch, dim, L, N, bias=True):
    return dict(
        u=rng.standard_normal((batch, dim, L)),
        delta=rng.standard_normal((batch, dim, L)) * 0.5,
        A=-rng.uniform(0.2, 3.0, size=(dim, N)),
        B=rng.standard_normal((batch, N, L)),
        C=rng.standard_normal((batch, N, L)),
        D=rng.standard_normal(dim),
        delta_bias=rng.uniform(-1.5, 0.5, size=dim) if bias else None,
    )


# ---------------------------------------------------------------- brute force
def _softplus_ref(x):
    return math.log1p(math.exp(x)) if x < 30 else x


def _brute(p, z=None, delta_softplus=True, reverse=False):
    """Materialised-kernel form of the scan, O(L^2 N) per channel:
    forward  y_t = sum_{k<=t} sum_n C[n,t] (prod_{k<j<=t} a_j,n) dt_k B[n,k] u_k + D u_t
    reverse  y_t = sum_{k>=t} sum_n C[n,t] (prod_{t<=j<k} a_j,n) dt_k B[n,k] u_k + D u_t
    with a_j,n = exp(dt_j A_n).  Plain Python loops, independent of the C code."""
    u, dl, A, B, C, D = p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"]
    bias = p.get("delta_bias")
    batch, dim, L = u.shape
    N = A.shape[1]
    out = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            dt = []
            for t in range(L):
                x = dl[b, d, t] + (bias[d] if bias is not None else 0.0)
                dt.append(_softplus_ref(x) if delta_softplus else x)
            for t in range(L):
                acc = 0.0
                ks = range(0, t + 1) if not reverse else range(t, L)
                for k in ks:
                    for n in range(N):
                        prod = 1.0
                        js = range(k + 1, t + 1) if not reverse else range(t, k)
                        for j in js:
                            prod *= math.exp(dt[j] * A[d, n])
                        acc += C[b, n, t] * prod * dt[k] * B[b, n, k] * u[b, d, k]
                y = acc + D[d] * u[b, d, t]
                if z is not None:
                    zz = z[b, d, t]
                    y *= zz / (1.0 + math.exp(-zz))
                out[b, d, t] = y
    return out


def _close(a, b, rel=1e-12):
    scale = max(1.0, float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= rel * scale, np.max(np.abs(a - b))


# ---------------------------------------------------------------- page numbers
def test_worked_example_gives_1_6(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    # two steps, one state, no softplus, zero bias, dt = 0.1, retention 0.5
    dt = 0.1
    A = np.array([[math.log(g["retention"]) / dt]])
    u = np.array([[[2.0, g["input"]]]])
    B = np.array([[[g["previous_state"] / (dt * 2.0), g["write"] / dt]]])
    C = np.ones((1, 1, 2))
    y = oracle.selective_scan(u, np.full((1, 1, 2), dt), A, B, C, np.zeros(1),
                              delta_softplus=False)
    assert y[0, 0, 0] == pytest.approx(g["previous_state"], abs=1e-14)
    assert y[0, 0, 1] == pytest.approx(g["new_state"], abs=1e-14)


def test_worked_example_through_softplus():
    # same update with softplus on: choose raw delta so that softplus gives 0.1
    raw = math.log(math.expm1(0.1))
    assert raw == pytest.approx(-2.2521684610440906, abs=1e-15)
    A = np.array([[math.log(0.5) / 0.1]])
    y = oracle.selective_scan(np.array([[[2.0, 3.0]]]), np.full((1, 1, 2), raw), A,
                              np.array([[[10.0, 2.0]]]), np.ones((1, 1, 2)), np.zeros(1))
    assert y[0, 0, 1] == pytest.approx(1.6, abs=1e-13)


def test_closed_form_constant_coefficients():
    # dt = 0.1, A = -1, B = u = C = 1, D = 0.5: h_t = dt (1 - a^(t+1)) / (1 - a)
    L = 300
    a = math.exp(-0.1)
    y = oracle.selective_scan(np.ones((1, 1, L)), np.full((1, 1, L), 0.1), np.array([[-1.0]]),
                              np.ones((1, 1, L)), np.ones((1, 1, L)), np.array([0.5]),
                              delta_softplus=False)[0, 0]
    expect = [0.1 * (1 - a ** (t + 1)) / (1 - a) + 0.5 for t in range(L)]
    _close(y, np.array(expect), 1e-13)
    printed = [0.6, 0.6904837418, 0.7723568171, 0.8464386392, 0.9134706438]
    assert np.allclose(y[:5], printed, atol=5e-11)
    assert y[-1] == pytest.approx(0.1 / (1 - a) + 0.5, rel=1e-12)   # -> 1.5508331945
    assert 0.1 / (1 - a) + 0.5 == pytest.approx(1.5508331945, abs=1e-10)


def test_softplus_known_values():
    # one step, one state, A = 0, B = C = u = 1, D = 0  =>  y_0 = softplus(delta + bias)
    def sp(x):
        return oracle.selective_scan(np.ones((1, 1, 1)), np.full((1, 1, 1), x), np.zeros((1, 1)),
                                     np.ones((1, 1, 1)), np.ones((1, 1, 1)), np.zeros(1))[0, 0, 0]
    assert sp(0.0) == pytest.approx(math.log(2.0), abs=1e-15)
    assert sp(math.log(math.e - 1.0)) == pytest.approx(1.0, abs=1e-15)
    assert sp(-30.0) == pytest.approx(9.357622968840175e-14, rel=1e-12)  # ~ e^-30
    assert sp(40.0) == pytest.approx(40.0, abs=1e-12)
    assert sp(800.0) == 800.0                                             # no overflow
    # bias enters before softplus
    y = oracle.selective_scan(np.ones((1, 1, 1)), np.full((1, 1, 1), 0.7), np.zeros((1, 1)),
                              np.ones((1, 1, 1)), np.ones((1, 1, 1)), np.zeros(1),
                              delta_bias=np.array([-0.7]))[0, 0, 0]
    assert y == pytest.approx(math.log(2.0), abs=1e-15)


def test_gate_known_value():
    # y = D u = 1 and z = ln 3  =>  SiLU(z) = ln3 * 3/4
    z = np.full((1, 1, 1), math.log(3.0))
    y = oracle.selective_scan(np.ones((1, 1, 1)), np.zeros((1, 1, 1)), np.zeros((1, 1)),
                              np.zeros((1, 1, 1)), np.zeros((1, 1, 1)), np.ones(1), z=z)[0, 0, 0]
    assert y == pytest.approx(0.75 * math.log(3.0), abs=1e-15)
    y0 = oracle.selective_scan(np.ones((1, 1, 1)), np.zeros((1, 1, 1)), np.zeros((1, 1)),
                               np.zeros((1, 1, 1)), np.zeros((1, 1, 1)), np.ones(1),
                               z=np.zeros((1, 1, 1)))[0, 0, 0]
    assert y0 == 0.0


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("gated", [False, True])
def test_brute_force(reverse, softplus, gated):
    rng = _rng(11 + 2 * reverse + 4 * softplus + 8 * gated)
    p = _rand_dir(rng, 2, 3, 7, 4)
    if not softplus:
        p["delta"] = rng.uniform(0.01, 0.6, size=p["u"].shape)
        p["delta_bias"] = rng.uniform(0.0, 0.1, size=3)
    z = rng.standard_normal(p["u"].shape) if gated else None
    got = oracle.selective_scan(**p, z=z, delta_softplus=softplus, reverse=reverse)
    want = _brute(p, z=z, delta_softplus=softplus, reverse=reverse)
    _close(got, want, 1e-12)


# ---------------------------------------------------------------- special cases
def test_zero_B_or_C_gives_skip_only():
    rng = _rng(3)
    p = _rand_dir(rng, 2, 5, 9, 3)
    for key in ("B", "C"):
        q = dict(p)
        q[key] = np.zeros_like(p[key])
        y = oracle.selective_scan(**q)
        assert np.array_equal(y, p["D"][None, :, None] * p["u"])


def test_zero_A_is_prefix_sum():
    rng = _rng(4)
    p = _rand_dir(rng, 2, 3, 11, 4)
    p["A"] = np.zeros_like(p["A"])
    p["delta"] = rng.uniform(0.05, 0.5, size=p["u"].shape)
    y = oracle.selective_scan(**p, delta_softplus=False)
    dt = p["delta"] + p["delta_bias"][None, :, None]
    w = dt[:, :, None, :] * p["B"][:, None, :, :] * p["u"][:, :, None, :]   # [b, d, n, t]
    h = np.cumsum(w, axis=-1)
    want = np.einsum("bdnt,bnt->bdt", h, p["C"]) + p["D"][None, :, None] * p["u"]
    _close(y, want, 1e-12)


def test_large_step_is_memoryless():
    rng = _rng(5)
    p = _rand_dir(rng, 1, 4, 10, 3)
    p["A"] = np.full_like(p["A"], -50.0)
    p["delta"] = np.full_like(p["u"], 2.0)
    p["delta_bias"] = None
    y = oracle.selective_scan(**p, delta_softplus=False)
    want = np.einsum("bnt,bnt->bt", p["C"], p["B"])[:, None, :] * 2.0 * p["u"] + p["D"][None, :, None] * p["u"]
    _close(y, want, 1e-12)


def test_linear_in_u():
    rng = _rng(6)
    p = _rand_dir(rng, 2, 3, 13, 4)
    u2 = rng.standard_normal(p["u"].shape)
    y1 = oracle.selective_scan(**p)
    y2 = oracle.selective_scan(**{**p, "u": u2})
    y12 = oracle.selective_scan(**{**p, "u": 2.0 * p["u"] - 3.0 * u2})
    _close(y12, 2.0 * y1 - 3.0 * y2, 1e-12)


@pytest.mark.parametrize("reverse", [False, True])
def test_causality(reverse):
    rng = _rng(7)
    p = _rand_dir(rng, 1, 3, 12, 4)
    y = oracle.selective_scan(**p, reverse=reverse)
    tp = 6
    q = {k: (v.copy() if v is not None else None) for k, v in p.items()}
    q["u"][:, :, tp] += 5.0
    q["delta"][:, :, tp] -= 1.0
    q["B"][:, :, tp] += 1.0
    y2 = oracle.selective_scan(**q, reverse=reverse)
    untouched = slice(0, tp) if not reverse else slice(tp + 1, None)
    touched = slice(tp, None) if not reverse else slice(0, tp + 1)
    assert np.array_equal(y[:, :, untouched], y2[:, :, untouched])
    assert np.all(np.abs(y[:, :, touched] - y2[:, :, touched]).max(axis=-1) > 0)


def test_reverse_equals_flip_scan_flip():
    rng = _rng(8)
    p = _rand_dir(rng, 2, 3, 10, 4)
    z = rng.standard_normal(p["u"].shape)
    yr = oracle.selective_scan(**p, z=z, reverse=True)
    f = dict(p)
    for k in ("u", "delta", "B", "C"):
        f[k] = p[k][..., ::-1]
    yf = oracle.selective_scan(**f, z=z[..., ::-1])[..., ::-1]
    assert np.array_equal(yr, yf)


# ---------------------------------------------------------------- bidirectional
def test_bidir_matches_two_directions():
    rng = _rng(9)
    fwd = _rand_dir(rng, 2, 4, 9, 4)
    bwd = _rand_dir(rng, 2, 4, 9, 4)
    z = rng.standard_normal(fwd["u"].shape)
    for s in (1.0, 0.5):
        got = oracle.bidir_scan(fwd, bwd, z=z, combine_scale=s)
        yf = _brute(fwd)
        yb = _brute(bwd, reverse=True)
        silu = z / (1.0 + np.exp(-z))
        _close(got, s * (yf + yb) * silu, 1e-12)


def test_bidir_palindrome_symmetry():
    rng = _rng(10)
    p = _rand_dir(rng, 1, 3, 9, 4)
    for k in ("u", "delta", "B", "C"):
        p[k] = 0.5 * (p[k] + p[k][..., ::-1])          # palindromic in t
    yf = oracle.selective_scan(**p)
    yb = oracle.selective_scan(**p, reverse=True)
    _close(yb, yf[..., ::-1], 1e-13)
    both = oracle.bidir_scan(p, p, combine_scale=1.0)
    _close(both, both[..., ::-1], 1e-13)


# ---------------------------------------------------------------- atrous routes
def test_atrous_routes_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "atrous_routes_4x6.json")))
    H, W = g["H"], g["W"]
    assert oracle.atrous_group_len(H, W) == g["group_len"]
    for k in range(4):
        rr, cc = oracle.atrous_route(H, W, k)
        assert list(rr * W + cc) == g["flat_order"][k]
    x = np.arange(H * W, dtype=np.float64).reshape(1, 1, H, W)
    s = oracle.atrous_gather(x)
    assert s.shape == (1, 4, 1, 6)
    assert s[0, :, 0, :].tolist() == [[float(v) for v in row] for row in g["flat_order"]]


def test_atrous_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "atrous_counts.json")))
    for c in g["cases"]:
        H, W = c["H"], c["W"]
        Lg = oracle.atrous_group_len(H, W)
        assert 4 * H * W == c["dense_visits"]
        assert 4 * Lg == c["sparse_visits"]
        assert 4 * Lg - H * W == c["padding_total"]
    for key, pads in g["per_group_padding"].items():
        H, W = map(int, key.split("x"))
        got = []
        for k in range(4):
            rr, cc = oracle.atrous_route(H, W, k)
            got.append(int(np.sum((rr >= H) | (cc >= W))))
        assert got == pads


@pytest.mark.parametrize("H,W", [(4, 6), (3, 5), (1, 1), (2, 3), (5, 2), (1, 7), (6, 1), (56, 56), (57, 57)])
def test_gather_scatter_identity(H, W):
    x = (np.arange(2 * 3 * H * W, dtype=np.float64) + 1.0).reshape(2, 3, H, W)
    s = oracle.atrous_gather(x)
    Lg = oracle.atrous_group_len(H, W)
    assert s.shape == (2, 4, 3, Lg)
    # every valid value appears once, pads are +0.0
    vals = s[s != 0]
    assert sorted(vals.tolist()) == sorted(x.ravel().tolist())
    assert int(np.sum(s == 0)) == 2 * 3 * (4 * Lg - H * W)
    assert not np.any(np.signbit(s[s == 0]))
    y = oracle.atrous_scatter(s, H, W)
    assert np.array_equal(y, x)                    # not four times the map


def test_es2d_impulse():
    # one nonzero u in group 1 at step m0; constant coefficients; identity-free scan
    H, W, N = 5, 6, 1
    Lg = oracle.atrous_group_len(H, W)
    dt, A, Bv, Cv, Dv, u0 = 0.3, -1.2, 0.7, 1.3, 0.25, 2.0
    k, m0 = 1, 1
    x = np.zeros((1, 1, H, W))
    rr, cc = oracle.atrous_route(H, W, k)
    x[0, 0, rr[m0], cc[m0]] = u0
    s = oracle.atrous_gather(x)                                   # [1, 4, 1, Lg]
    u = s.reshape(4, 1, Lg)
    y = oracle.selective_scan(u, np.full((4, 1, Lg), dt), np.array([[A]]),
                              np.full((4, N, Lg), Bv), np.full((4, N, Lg), Cv), np.array([Dv]),
                              delta_softplus=False)
    out = oracle.atrous_scatter(y.reshape(1, 4, 1, Lg), H, W)[0, 0]
    a = math.exp(dt * A)
    want = np.zeros((H, W))
    for t in range(Lg):
        r, c = rr[t], cc[t]
        if r >= H or c >= W or t < m0:
            continue
        v = Cv * a ** (t - m0) * dt * Bv * u0
        if t == m0:
            v += Dv * u0
        want[r, c] = v
    _close(out, want, 1e-14)
    # every coordinate outside group 1 is exactly zero
    mask = np.ones((H, W), dtype=bool)
    mask[rr[(rr < H) & (cc < W)], cc[(rr < H) & (cc < W)]] = False
    assert np.all(out[mask] == 0.0)


# ---------------------------------------------------------------- pooling
def test_mean_pool_integer_values():
    rng = _rng(12)
    u = rng.integers(-8, 9, size=(2, 3, 4, 8)).astype(np.float64)
    p0 = oracle.mean_pool(u, 0)
    p1 = oracle.mean_pool(u, 1)
    assert p0.shape == (2, 3, 4) and p1.shape == (2, 3, 8)
    assert np.array_equal(p0 * 8, u.sum(axis=3))
    assert np.array_equal(p1 * 4, u.sum(axis=2))


@pytest.mark.parametrize("axis", [0, 1])
def test_pool_repeat_identity_on_constant_axis(axis):
    rng = _rng(13 + axis)
    batch, dim, H, W, N = 2, 3, 4, 6, 2
    Lp = H if axis == 0 else W
    base = rng.integers(-8, 9, size=(batch, dim, Lp)).astype(np.float64)
    u = np.repeat(base[:, :, :, None], W, axis=3) if axis == 0 else np.repeat(base[:, :, None, :], H, axis=2)
    d = dict(u=u, delta=rng.standard_normal((batch, dim, Lp)), A=-np.ones((dim, N)),
             B=np.zeros((batch, N, Lp)), C=rng.standard_normal((batch, N, Lp)), D=np.ones(dim))
    out = oracle.pool_scan_repeat(d, None, combine_scale=1.0, pool_axis=axis)
    assert np.array_equal(out, u)
    out2 = oracle.pool_scan_repeat(d, d, combine_scale=0.5, pool_axis=axis)
    assert np.array_equal(out2, u)


def test_pool_width_one_is_plain_bidir_scan():
    rng = _rng(14)
    batch, dim, H, N = 2, 3, 7, 4
    fwd = _rand_dir(rng, batch, dim, H, N)
    bwd = _rand_dir(rng, batch, dim, H, N)
    z = rng.standard_normal((batch, dim, H, 1))
    want = oracle.bidir_scan(fwd, bwd, z=z[..., 0], combine_scale=0.5)
    f4 = {**fwd, "u": fwd["u"][..., None]}
    b4 = {**bwd, "u": bwd["u"][..., None]}
    got = oracle.pool_scan_repeat(f4, b4, z=z, combine_scale=0.5, pool_axis=0)
    _close(got[..., 0], want, 1e-14)


@pytest.mark.parametrize("axis", [0, 1])
def test_pool_repeat_broadcast_axis(axis):
    # the gate is per full-resolution element; the scanned value is per pooled index
    rng = _rng(15 + axis)
    batch, dim, H, W, N = 1, 2, 3, 5, 2
    Lp = H if axis == 0 else W
    f = dict(u=rng.standard_normal((batch, dim, H, W)), delta=rng.standard_normal((batch, dim, Lp)),
             A=-rng.uniform(0.5, 2, (dim, N)), B=rng.standard_normal((batch, N, Lp)),
             C=rng.standard_normal((batch, N, Lp)), D=rng.standard_normal(dim))
    z = rng.standard_normal((batch, dim, H, W))
    out = oracle.pool_scan_repeat(f, None, z=z, pool_axis=axis)
    pooled = f["u"].mean(axis=3 if axis == 0 else 2)
    y = _brute({**f, "u": pooled})
    silu = z / (1 + np.exp(-z))
    want = (y[:, :, :, None] if axis == 0 else y[:, :, None, :]) * silu
    _close(out, want, 1e-12)


# ---------------------------------------------------------------- SS2D
def _ss2d_dirs(rng, batch, dim, H, W, N):
    return [dict(delta=rng.standard_normal((batch, dim, H * W)) * 0.5,
                 A=-rng.uniform(0.2, 3.0, size=(dim, N)),
                 B=rng.standard_normal((batch, N, H * W)),
                 C=rng.standard_normal((batch, N, H * W)),
                 D=rng.standard_normal(dim),
                 delta_bias=rng.uniform(-1.5, 0.5, size=dim)) for _ in range(4)]


def test_ss2d_brute_force():
    # four traversals written out here as pixel lists: left-to-right rows,
    # their reverse, top-to-bottom columns, their reverse; each scanned by the
    # materialised-kernel brute force and summed back at its pixels
    rng = _rng(41)
    batch, dim, H, W, N = 2, 2, 2, 3, 3
    u = rng.standard_normal((batch, dim, H, W))
    z = rng.standard_normal((batch, dim, H, W))
    dirs = _ss2d_dirs(rng, batch, dim, H, W, N)
    rows = [(i, j) for i in range(H) for j in range(W)]
    cols = [(i, j) for j in range(W) for i in range(H)]
    want = np.zeros((batch, dim, H, W))
    for k in range(4):
        order = rows if k < 2 else cols
        uk = np.stack([u[:, :, i, j] for (i, j) in order], axis=-1)
        yk = _brute(dict(dirs[k], u=uk), reverse=(k % 2 == 1))
        for t, (i, j) in enumerate(order):
            want[:, :, i, j] += yk[:, :, t]
    want = 0.5 * want * z / (1.0 + np.exp(-z))
    got = oracle.ss2d_scan(u, dirs, z=z, combine_scale=0.5)
    _close(got, want, 1e-12)


@pytest.mark.parametrize("H,W", [(1, 7), (6, 1)])
def test_ss2d_line_is_twice_bidir(H, W):
    # on a single row or column both traversal orders coincide: with the
    # column directions given the row directions' parameters, SS2D is twice
    # the bidirectional scan
    rng = _rng(42 + H)
    u = rng.standard_normal((1, 3, H, W))
    d = _ss2d_dirs(rng, 1, 3, H, W, 4)
    dirs = [d[0], d[1], d[0], d[1]]
    got = oracle.ss2d_scan(u, dirs)
    flat = u.reshape(1, 3, H * W)
    want = 2.0 * oracle.bidir_scan(dict(d[0], u=flat), dict(d[1], u=flat))
    _close(got.reshape(1, 3, H * W), want, 1e-12)


def test_ss2d_transpose_symmetry():
    # the column traversals of u are the row traversals of u transposed
    rng = _rng(43)
    u = rng.standard_normal((2, 2, 3, 5))
    z = rng.standard_normal(u.shape)
    d = _ss2d_dirs(rng, 2, 2, 3, 5, 4)
    got = oracle.ss2d_scan(u, d, z=z)
    tr = oracle.ss2d_scan(u.transpose(0, 1, 3, 2), [d[2], d[3], d[0], d[1]], z=z.transpose(0, 1, 3, 2))
    _close(got, tr.transpose(0, 1, 3, 2), 1e-12)


# ---------------------------------------------------------------- zero-order hold
# ("Norm or Direction?" page, section 3, eq. 1-2; Vim page, "A state retains,
# writes, and reads": the exact zero-order-hold input coefficient)
def _van_loan(a, dt):
    """Exact discretisation of h' = a h + b u over one step of length dt with
    b u held constant: exp([[a, 1], [0, 0]] dt) = [[exp(a dt), g], [0, 1]],
    g = integral_0^dt exp(a s) ds (Van Loan's block-matrix exponential,
    evaluated by scipy's Pade expm)."""
    from scipy.linalg import expm
    m = expm(np.array([[a * dt, dt], [0.0, 0.0]]))
    return m[0, 0], m[0, 1]


def _zoh_ref(p, z=None, delta_softplus=True, reverse=False):
    """Sequential scan with per-step (Abar, Bbar) from _van_loan, plain loops."""
    u, dl, A, B, C, D = p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"]
    bias = p.get("delta_bias")
    batch, dim, L = u.shape
    N = A.shape[1]
    out = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            h = [0.0] * N
            order = range(L - 1, -1, -1) if reverse else range(L)
            for t in order:
                x = dl[b, d, t] + (bias[d] if bias is not None else 0.0)
                dt = _softplus_ref(x) if delta_softplus else x
                acc = 0.0
                for n in range(N):
                    abar, g = _van_loan(A[d, n], dt)
                    h[n] = abar * h[n] + g * B[b, n, t] * u[b, d, t]
                    acc += C[b, n, t] * h[n]
                y = acc + D[d] * u[b, d, t]
                if z is not None:
                    y *= z[b, d, t] / (1.0 + math.exp(-z[b, d, t]))
                out[b, d, t] = y
    return out


@pytest.mark.parametrize("reverse", [False, True])
def test_zoh_van_loan(reverse):
    rng = _rng(60 + reverse)
    p = _rand_dir(rng, 2, 3, 9, 4)
    z = rng.standard_normal(p["u"].shape)
    got = oracle.selective_scan(**p, z=z, reverse=reverse, zoh=True)
    _close(got, _zoh_ref(p, z=z, reverse=reverse), 1e-12)
    # and it is not the released recurrence
    assert np.max(np.abs(got - oracle.selective_scan(**p, z=z, reverse=reverse))) > 1e-3


def test_zoh_small_step_keeps_digits():
    # dt A = -2e-7: exp(dt A) - 1 would lose about 9 of fp64's 16 digits; the
    # comparison is relative to this channel's own (tiny) output
    rng = _rng(62)
    p = _rand_dir(rng, 1, 1, 6, 3, bias=False)
    p["delta"] = np.full((1, 1, 6), 1e-7)
    p["A"] = np.array([[-2.0, -0.5, -3.0]])
    p["D"] = np.zeros(1)
    got = oracle.selective_scan(**p, delta_softplus=False, zoh=True)
    ref = _zoh_ref(p, delta_softplus=False)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_zoh_constant_input_closed_form():
    # constant dt, B, u, C: the zero-order hold is exact, so h after t+1 steps
    # is the ODE solution h(T) = (b u / a) (exp(a T) - 1) at T = (t+1) dt
    L, N, dt = 12, 3, 0.3
    a = np.array([-0.5, -1.0, -2.5])
    bv, cv, uv, Dv = np.array([0.7, -1.2, 2.0]), np.array([1.5, 0.4, -0.8]), 1.3, 0.25
    p = dict(u=np.full((1, 1, L), uv), delta=np.full((1, 1, L), dt), A=a[None, :],
             B=np.repeat(bv[None, :, None], L, axis=2), C=np.repeat(cv[None, :, None], L, axis=2),
             D=np.array([Dv]), delta_bias=None)
    got = oracle.selective_scan(**p, delta_softplus=False, zoh=True)[0, 0]
    T = dt * np.arange(1, L + 1)
    h = (bv * uv / a)[None, :] * np.expm1(a[None, :] * T[:, None])
    _close(got, h @ cv + Dv * uv, 1e-12)


def test_zoh_zero_A_is_euler():
    # the coefficient's limit at A = 0 is dt: both discretisations coincide,
    # and at A = -1e-200 they agree to rounding
    rng = _rng(63)
    p = _rand_dir(rng, 2, 2, 7, 3)
    p["A"] = np.zeros_like(p["A"])
    assert np.array_equal(oracle.selective_scan(**p, zoh=True), oracle.selective_scan(**p))
    p["A"] = np.full_like(p["A"], -1e-200)
    _close(oracle.selective_scan(**p, zoh=True), oracle.selective_scan(**p), 1e-14)


def test_zoh_reaches_bidir_pool_and_ss2d():
    rng = _rng(64)
    f, b = _rand_dir(rng, 1, 2, 6, 3), _rand_dir(rng, 1, 2, 6, 3)
    z = rng.standard_normal(f["u"].shape)
    got = oracle.bidir_scan(f, b, z=z, combine_scale=0.5, zoh=True)
    want = 0.5 * (_zoh_ref(f) + _zoh_ref(b, reverse=True)) * z / (1.0 + np.exp(-z))
    _close(got, want, 1e-12)
    # pooled: mean over W (axis 0), scan, repeat
    H, W = 3, 4
    pf = _rand_dir(rng, 1, 2, H, 3)
    pf["u"] = rng.standard_normal((1, 2, H, W))
    got = oracle.pool_scan_repeat(pf, None, zoh=True)
    want = _zoh_ref(dict(pf, u=pf["u"].mean(axis=3)))
    _close(got, np.repeat(want[..., None], W, axis=3), 1e-12)
    # SS2D on a single row: every traversal is a plain row scan
    u = rng.standard_normal((1, 2, 1, 5))
    d = _ss2d_dirs(rng, 1, 2, 1, 5, 3)
    flat = u.reshape(1, 2, 5)
    want = sum(_zoh_ref(dict(d[k], u=flat), reverse=k % 2 == 1) for k in range(4))
    _close(oracle.ss2d_scan(u, d, zoh=True).reshape(1, 2, 5), want, 1e-12)


# ---------------------------------------------------------------- causal conv1d + SiLU
# (Vim page, "Inside the released Vim block": depthwise, kernel four, causal,
# then SiLU; the backward branch convolves the reversed sequence)
def _silu(v):
    return v / (1.0 + np.exp(-v))


@pytest.mark.parametrize("reverse", [False, True])
def test_conv_matches_torch_conv1d(reverse):
    import torch
    rng = _rng(70 + reverse)
    batch, dim, L = 2, 5, 11
    x, w, b = rng.standard_normal((batch, dim, L)), rng.standard_normal((dim, 4)), rng.standard_normal(dim)
    xt = torch.from_numpy(x)
    if reverse:
        xt = torch.flip(xt, dims=[-1])
    v = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(b),
                                   padding=3, groups=dim)[..., :L]
    want = torch.nn.functional.silu(v)
    if reverse:
        want = torch.flip(want, dims=[-1])
    _close(oracle.causal_conv1d_silu(x, w, b, reverse=reverse), want.numpy(), 1e-13)


def test_conv_matches_numpy_convolve():
    rng = _rng(72)
    x, w = rng.standard_normal((1, 3, 9)), rng.standard_normal((3, 4))
    got = oracle.causal_conv1d_silu(x, w)
    for d in range(3):
        _close(got[0, d], _silu(np.convolve(x[0, d], w[d, ::-1])[:9]), 1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_conv_impulse_response(reverse):
    # a unit impulse at t0 reaches t0 (weight w[3]) and the next three steps
    # in scan order (w[2], w[1], w[0]); every other token sees only the bias
    L, t0, bias = 10, 4, 0.3
    w = np.array([[0.5, -1.25, 2.0, 0.75]])
    x = np.zeros((1, 1, L))
    x[0, 0, t0] = 1.0
    got = oracle.causal_conv1d_silu(x, w, np.array([bias]), reverse=reverse)[0, 0]
    want = np.full(L, _silu(bias))
    for j in range(4):
        t = t0 - j if reverse else t0 + j
        want[t] = _silu(bias + w[0, 3 - j])
    _close(got, want, 1e-14)


def test_conv_first_tokens_see_zero_padding():
    # the first three tokens have fewer than four real predecessors: the
    # missing ones count as zero (left padding), so a constant input ramps up
    x = np.ones((1, 1, 6))
    w = np.array([[1.0, 2.0, 4.0, 8.0]])
    got = oracle.causal_conv1d_silu(x, w)[0, 0]
    _close(got, _silu(np.array([8.0, 12.0, 14.0, 15.0, 15.0, 15.0])), 1e-14)


@pytest.mark.parametrize("H,W", [(56, 56), (57, 57), (5, 8), (1, 1)])
def test_atrous_gather_and_scatter_are_adjoint(H, W):
    """<gather(x), s> = <x, scatter(s)>: gather is a permutation into the
    streams with zero padding, scatter its transpose on the valid map, so
    the backward of either is the other (ES2D training composes from them)."""
    rng = np.random.default_rng(H * 100 + W)
    x = rng.standard_normal((2, 3, H, W))
    st = rng.standard_normal((2, 4, 3, oracle.atrous_group_len(H, W)))
    lhs = float(np.sum(oracle.atrous_gather(x) * st))
    rhs = float(np.sum(x * oracle.atrous_scatter(st, H, W)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))

