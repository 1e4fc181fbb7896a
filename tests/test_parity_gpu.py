"""GPU parity of every C-ABI entry point against the fp64 CPU oracle.

Scan outputs must agree within max relative error 1e-4 (fp32) / 2e-2 (bf16
inputs), measured as max |got - ref| / max(|ref|, 0.1 rms(ref)); gather and
scatter must be bit-exact.  Small cases span several tiles, several row
blocks and ragged tails; full-size cases check sampled rows of the workloads
at their real shapes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import selective_scan_fwd_amd as vm
from selective_scan_fwd_amd import workloads as wl

from _helpers import BF16_TOL, FP32_TOL, assert_close, bits_equal, host, host_dir, sub_dir

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _case(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if DEV is None:
        pytest.fail("GPU test run without a visible GPU")
    vm.load_library()


# ---------------------------------------------------------------- one direction
@pytest.mark.parametrize("batch,dim,L,N", [(1, 1, 1, 16), (2, 130, 77, 16), (3, 64, 8, 16),
                                           (2, 70, 33, 5), (1, 96, 197, 1), (2, 33, 150, 16)])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("bc_layout", ["token", "dense"])
def test_single_fp32(batch, dim, L, N, reverse, gated, bc_layout):
    _case(f"single fp32 b{batch} d{dim} L{L} N{N} rev{reverse} gated{gated} bc {bc_layout}")
    p, z = wl.single_inputs(100 + L, batch, dim, L, N, device=DEV, gated=gated, perturb=True,
                            bc_layout=bc_layout)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), reverse=reverse)
    assert_close(host(out), ref, FP32_TOL, "single")


# Sequence-parallel scan: one direction with few row blocks (and 32 to 256
# steps) runs with each lane on a sub-chunk of ceil(L / 64) steps and the
# lanes' (P, g) carries combined by a lane scan.  L 32 -> 1 step per lane
# (lanes 32.. idle), 65 -> 2 (lanes 33.. idle), 197 -> 4 (a ragged last
# lane), 256 -> 4 (every lane full); 257 is past the staged row (the
# one-wave-per-row-block kernel); dstate 5 as well.
@pytest.mark.parametrize("L", [32, 65, 197, 256, 257])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("N", [16, 5])
def test_single_chunked(L, reverse, N):
    _case(f"single chunked L{L} rev{reverse} N{N}")
    p, z = wl.single_inputs(150 + L + N, 1, 70, L, N, device=DEV, perturb=True)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), reverse=reverse)
    assert_close(host(out), ref, FP32_TOL, "single chunked")


@pytest.mark.parametrize("L", [33, 77])
@pytest.mark.parametrize("reverse", [False, True])
def test_single_many_rows_unchunked(L, reverse):
    """1024 row blocks (batch 64 x 16 blocks of 16 channels): the one-wave-per-
    row-block kernel, with tiles of 16 steps and a ragged tail."""
    _case(f"single many rows L{L} rev{reverse}")
    p, z = wl.single_inputs(160 + L, 64, 256, L, device=DEV, perturb=True)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), reverse=reverse)
    assert_close(host(out), ref, FP32_TOL, "single many rows")


def test_single_no_softplus_and_no_bias():
    _case("single no softplus")
    p, z = wl.single_inputs(5, 2, 70, 45, device=DEV)
    p["delta"] = torch.rand_like(p["delta"]) * 0.2
    p["delta_bias"] = None
    out = vm.vm_selective_scan_fwd(**p, z=z, delta_softplus=False)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), delta_softplus=False)
    assert_close(host(out), ref, FP32_TOL, "no softplus")


def test_single_extreme_steps():
    # softplus far in both tails: dt ~ e^-30 (no update) and dt ~ 30 (memoryless)
    _case("single extreme steps")
    p, z = wl.single_inputs(6, 1, 64, 40, device=DEV)
    p["delta"][:, :, ::3] = -30.0
    p["delta"][:, :, 1::3] = 30.0
    out = vm.vm_selective_scan_fwd(**p, z=z)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z))
    assert_close(host(out), ref, FP32_TOL, "extreme")


def test_single_bf16():
    _case("single bf16")
    p, z = wl.single_inputs(7, 2, 100, 90, device=DEV, dtype=torch.bfloat16, perturb=True)
    out = vm.vm_selective_scan_fwd(**p, z=z)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref = oracle.selective_scan(**host_dir(p), z=host(z))
    assert_close(host(out), ref, BF16_TOL, "single bf16")


# ---------------------------------------------------------------- bidirectional
# Shapes chosen to cover: one tile (joint midpoint), odd / even tile counts,
# the LDS exchange (8-step tiles) and the global exchange (16-step tiles,
# long L), with many and few row blocks.
# L = 552 is the longest sequence of the on-chip exchange (its LDS block is
# 16 x 552 floats); 553 and 600 take the global exchange through a pool
# buffer, 576 (fp32, L % 32 == 0) parks in `out` itself.
BIDIR_CASES = [
    (1, 1, 1), (2, 70, 2), (2, 70, 16), (2, 70, 77), (2, 130, 197), (2, 70, 300),
    (512, 64, 20), (512, 64, 197), (256, 128, 300),
    (2, 40, 456), (2, 40, 552), (2, 40, 553), (1, 33, 600), (2, 20, 576),
]


@pytest.mark.parametrize("batch,dim,L", BIDIR_CASES)
@pytest.mark.parametrize("bc_layout", ["token", "dense"])
def test_bidir_fp32(batch, dim, L, bc_layout):
    _case(f"bidir fp32 b{batch} d{dim} L{L} bc {bc_layout}")
    fwd, bwd, z = wl.bidir_inputs(200 + L, batch, dim, L, device=DEV, perturb=True,
                                  bc_layout=bc_layout)
    for scale in (1.0, 0.5):
        out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=scale)
        torch.cuda.synchronize()
        ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z), combine_scale=scale)
        assert_close(host(out), ref, FP32_TOL, f"bidir s={scale}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [9, 37])
def test_bidir_two_row_blocks_per_workgroup(dtype, L):
    """Enough row blocks (83 x 25 = 2075, odd) for workgroups of two row
    blocks: the last workgroup's second row block is empty, and the last row
    block of each batch row is partial (dim 397 = 24 x 16 + 13)."""
    _case(f"bidir two row blocks per workgroup {dtype} L{L}")
    batch, dim = 83, 397
    fwd, bwd, z = wl.bidir_inputs(400 + L, batch, dim, L, device=DEV, dtype=dtype, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z), combine_scale=0.5)
    assert_close(host(out), ref, FP32_TOL if dtype == torch.float32 else BF16_TOL, "two row blocks")


def test_bidir_ungated_small_dstate():
    _case("bidir ungated N=3")
    fwd, bwd, _ = wl.bidir_inputs(9, 2, 66, 41, dstate=3, device=DEV, gated=False, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=None, combine_scale=0.5)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=None, combine_scale=0.5)
    assert_close(host(out), ref, FP32_TOL, "bidir N=3")


@pytest.mark.parametrize("L", [50, 333])
@pytest.mark.parametrize("bc_layout", ["token", "dense"])
def test_bidir_bf16(L, bc_layout):
    _case(f"bidir bf16 L{L} bc {bc_layout}")
    fwd, bwd, z = wl.bidir_inputs(11 + L, 2, 100, L, device=DEV, dtype=torch.bfloat16, perturb=True,
                                  bc_layout=bc_layout)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z))
    assert_close(host(out), ref, BF16_TOL, "bidir bf16")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_projection_split_layout(dtype):
    # B and C as the page's projection yields them: slices of one token-major
    # [batch, L, rank + 2N] tensor, passed as transposed views (token stride 44)
    _case(f"projection-split B/C {dtype}")
    batch, dim, L, N, rank = 2, 96, 70, 16, 12
    fwd, bwd, z = wl.bidir_inputs(14, batch, dim, L, device=DEV, dtype=dtype, perturb=True)
    for p in (fwd, bwd):
        proj = torch.randn((batch, L, rank + 2 * N), device=DEV).to(dtype)
        p["B"] = proj[:, :, rank:rank + N].transpose(1, 2)
        p["C"] = proj[:, :, rank + N:].transpose(1, 2)
        assert p["B"].stride() == (L * (rank + 2 * N), 1, rank + 2 * N)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z))
    assert_close(host(out), ref, FP32_TOL if dtype == torch.float32 else BF16_TOL, "proj split")


def test_bidir_matches_two_single_calls():
    # the fused kernel equals (fwd scan + reverse scan) * scale * gate from the
    # one-direction entry point, within rounding
    _case("bidir vs two singles")
    fwd, bwd, z = wl.bidir_inputs(12, 2, 64, 90, device=DEV, perturb=True)
    yf = vm.vm_selective_scan_fwd(**fwd)
    yb = vm.vm_selective_scan_fwd(**bwd, reverse=True)
    both = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    zz = host(z)
    comp = 0.5 * (host(yf) + host(yb)) * (zz / (1 + np.exp(-zz)))
    assert_close(host(both), comp, FP32_TOL, "fused vs composed")


def test_deterministic():
    _case("determinism")
    fwd, bwd, z = wl.bidir_inputs(13, 4, 128, 197, device=DEV)
    a = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    b = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------- atrous
# Vector paths: (8, 6) gathers with 4-value accesses but scatters per value
# (W % 4 != 0); (6, 8), (7, 8), (56, 56), (100, 100) take them both ways,
# (7, 8) with a padded row; (129, 130) exceeds the LDS staging limit.
SHAPES = [(4, 6), (3, 5), (1, 1), (2, 3), (5, 2), (1, 7), (6, 1), (56, 56), (57, 57), (130, 9),
          (8, 6), (6, 8), (7, 8), (100, 100), (129, 130)]


@pytest.mark.parametrize("H,W", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_atrous_bit_exact(H, W, dtype):
    _case(f"atrous {H}x{W} {dtype}")
    g = wl.generator(300 + H * 31 + W, DEV)
    x = torch.randn((2, 3, H, W), generator=g, device=DEV).to(dtype)
    s = vm.vm_atrous_gather(x)
    y = vm.vm_atrous_scatter(s, H, W)
    torch.cuda.synchronize()
    ref = oracle.atrous_gather(host(x))
    assert bits_equal(s, ref)                              # pads are +0.0, values copied
    assert torch.equal(y.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    # scatter alone against the oracle on arbitrary stream contents
    s2 = torch.randn(s.shape, generator=g, device=DEV).to(dtype)
    y2 = vm.vm_atrous_scatter(s2, H, W)
    torch.cuda.synchronize()
    assert bits_equal(y2, oracle.atrous_scatter(host(s2), H, W))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_atrous_misaligned_views(dtype):
    """Tensors starting one element past an aligned address take the per-value
    paths; the results are bit-identical to the aligned call's."""
    _case(f"atrous misaligned {dtype}")
    H = W = 56
    g = wl.generator(311, DEV)
    x = torch.randn((2, 3, H, W), generator=g, device=DEV).to(dtype)
    ref_s = vm.vm_atrous_gather(x)
    ref_y = vm.vm_atrous_scatter(ref_s, H, W)
    xb = torch.empty(x.numel() + 1, device=DEV, dtype=dtype)
    xm = xb[1:].view(x.shape)
    xm.copy_(x)
    sb = torch.empty(ref_s.numel() + 1, device=DEV, dtype=dtype)
    sm = sb[1:].view(ref_s.shape)
    vm.vm_atrous_gather(xm, out=sm)
    yb = torch.empty(x.numel() + 1, device=DEV, dtype=dtype)
    ym = yb[1:].view(x.shape)
    vm.vm_atrous_scatter(sm, H, W, out=ym)
    torch.cuda.synchronize()
    assert bits_equal(sm, host(ref_s))
    assert bits_equal(ym, host(ref_y))


def test_atrous_pad_is_positive_zero():
    _case("atrous pad sign")
    x = -torch.ones((1, 1, 3, 5), device=DEV)
    s = vm.vm_atrous_gather(x)
    torch.cuda.synchronize()
    sv = host(s)
    pads = sv == 0
    assert int(pads.sum()) == 9
    assert not np.any(np.signbit(sv[pads]))


@pytest.mark.parametrize("H,W", [(7, 10), (56, 56)])
def test_es2d_pipeline(H, W):
    _case(f"es2d pipeline {H}x{W}")
    batch, ch = 2, 70
    x, p = wl.es2d_inputs(400 + H, batch, ch, H, W, device=DEV, perturb=True)
    s = vm.vm_atrous_gather(x)
    Lg = s.shape[-1]
    y = vm.vm_selective_scan_fwd(s.reshape(4 * batch, ch, Lg), **p)
    out = vm.vm_atrous_scatter(y.reshape(batch, 4, ch, Lg), H, W)
    torch.cuda.synchronize()
    hs = oracle.atrous_gather(host(x))
    hy = oracle.selective_scan(hs.reshape(4 * batch, ch, Lg), **host_dir(p))
    ref = oracle.atrous_scatter(hy.reshape(batch, 4, ch, Lg), H, W)
    assert_close(host(out), ref, FP32_TOL, "es2d")


# ---------------------------------------------------------------- pooled
# (12, 10): scalar pooling path; (12, 32) and (40, 8): four-wide path with
# 8 and 2 threads per grid row and a ragged last pass.
@pytest.mark.parametrize("H,W", [(12, 10), (12, 32), (40, 8)])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("gated", [True, False])
def test_pool_scan_repeat_fp32(H, W, axis, bidir, gated):
    _case(f"pool {H}x{W} axis{axis} bidir{bidir} gated{gated}")
    fwd, bwd, z = wl.fastvim_inputs(500 + axis, 2, 70, H, W, axis, device=DEV, perturb=True)
    out = vm.vm_pool_scan_repeat(fwd, bwd if bidir else None, z=z if gated else None,
                                 combine_scale=0.5, pool_axis=axis)
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(bwd) if bidir else None,
                                  z=host(z) if gated else None, combine_scale=0.5, pool_axis=axis)
    assert_close(host(out), ref, FP32_TOL, "pool")


@pytest.mark.parametrize("axis", [0, 1])
def test_pool_repeat_indexing_bit_exact(axis):
    # integer-valued u, B = 0, D = 1, no gate: out = s * (mean_f + mean_b),
    # exact in fp32 and fp64 (sums < 2^24, division by a power of two)
    _case(f"pool bit-exact axis{axis}")
    H, W = 8, 16
    fwd, bwd, _ = wl.fastvim_inputs(600 + axis, 2, 3, H, W, axis, device=DEV)
    for p in (fwd, bwd):
        p["u"] = torch.randint(-8, 9, p["u"].shape, device=DEV).float()
        p["B"] = torch.zeros_like(p["B"])
        p["D"] = torch.ones_like(p["D"])
    out = vm.vm_pool_scan_repeat(fwd, bwd, z=None, combine_scale=0.5, pool_axis=axis)
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(bwd), z=None, combine_scale=0.5,
                                  pool_axis=axis)
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("H,W", [(12, 10), (6, 5), (3, 6), (8, 16)])
@pytest.mark.parametrize("axis", [0, 1])
def test_pool_repeat_indexing_bit_exact_any_extent(H, W, axis):
    """Pool and repeat indexing on every path (W = 10, 5, 6: one value per
    access; W = 16: four-wide), with pooled extents that are not powers of
    two.  Each pooled line is an integer c in [-8, 8] plus integer offsets
    that sum to zero, so its sum is exactly w c on both sides and the mean is
    exactly c: the device's sum x fl(1/w) rounds to c because w fl(1/w) is
    within 2^-25 of 1 for these w (checked below in fp32), and the oracle
    divides exactly.  With B = 0 and D = 1 the scan returns the mean, so an
    element summed into the wrong line, or repeated along the wrong axis,
    changes a value."""
    _case(f"pool bit-exact {H}x{W} axis{axis}")
    w = W if axis == 0 else H
    assert abs(w * float(np.float32(1.0 / w)) - 1.0) <= 2.0 ** -25
    gen = np.random.default_rng(650 + 10 * H + W + axis)
    fwd, bwd, _ = wl.fastvim_inputs(650 + axis, 2, 3, H, W, axis, device=DEV)
    for p in (fwd, bwd):
        batch, dim = p["u"].shape[:2]
        lines = H if axis == 0 else W
        c = gen.integers(-8, 9, size=(batch, dim, lines, 1))
        off = gen.integers(-4, 5, size=(batch, dim, lines, w))
        off[..., -1] -= off.sum(axis=-1)
        vals = (c + off).astype(np.float32)          # [batch, dim, line, position in line]
        if axis == 1:
            vals = vals.transpose(0, 1, 3, 2)          # lines are columns
        p["u"] = torch.from_numpy(np.ascontiguousarray(vals)).to(DEV)
        p["B"] = torch.zeros_like(p["B"])
        p["D"] = torch.ones_like(p["D"])
    out = vm.vm_pool_scan_repeat(fwd, bwd, z=None, combine_scale=0.5, pool_axis=axis)
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(bwd), z=None, combine_scale=0.5, pool_axis=axis)
    assert bits_equal(out, ref)


@pytest.mark.parametrize("H,W,axis", [(16, 12, 1), (20, 16, 0), (20, 16, 1)])
def test_pool_bf16(H, W, axis):
    _case(f"pool bf16 {H}x{W} axis{axis}")
    fwd, bwd, z = wl.fastvim_inputs(700, 2, 70, H, W, axis, device=DEV, dtype=torch.bfloat16)
    out = vm.vm_pool_scan_repeat(fwd, bwd, z=z, pool_axis=axis)
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(bwd), z=host(z), pool_axis=axis)
    assert_close(host(out), ref, BF16_TOL, "pool bf16")


@pytest.mark.parametrize("H,W", [(6, 8), (5, 3)])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("zoh", [False, True])
def test_pool_scan_repeat_bwd(H, W, axis, bidir, gated, zoh):
    # zoh: the pooled scans discretised by zero-order hold (FastVim summary,
    # "Methodology"; "Norm or Direction?" page, section 3, eq. 2)
    _case(f"pool bwd {H}x{W} axis{axis} bidir{bidir} gated{gated} zoh{zoh}")
    fwd, bwd, z = wl.fastvim_inputs(4000 + axis, 2, 40, H, W, axis, device=DEV, perturb=True)
    dout = torch.randn(z.shape, generator=wl.generator(4010 + axis, DEV), device=DEV)
    gf, gb, dz = vm.vm_pool_scan_repeat_bwd(fwd, dout, bwd=bwd if bidir else None,
                                            z=z if gated else None, combine_scale=0.5, pool_axis=axis, zoh=zoh)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.pool_scan_repeat_grad(host_dir(fwd), host_dir(bwd) if bidir else None,
                                                 host(dout), z=host(z) if gated else None,
                                                 combine_scale=0.5, pool_axis=axis, zoh=zoh)
    for got, want, tag in ((gf, wf, "fwd"), (gb, wb, "bwd")):
        if want is None:
            assert got is None
            continue
        for k in _GRAD_KEYS:
            assert_close(host(got[k]), want[k], FP32_TOL, f"{tag} d{k}")
    if gated:
        assert_close(host(dz), wdz, FP32_TOL, "dz")
    else:
        assert dz is None


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pool_scan_repeat_bwd_long_pooled_axis(dtype):
    """A pooled length past the on-chip exchange (600 > 552), bf16 inputs."""
    _case(f"pool bwd long pooled axis {dtype}")
    fwd, bwd, z = wl.fastvim_inputs(4100, 1, 16, 600, 3, 0, device=DEV, dtype=dtype, perturb=True)
    dout = torch.randn(z.shape, generator=wl.generator(4101, DEV), device=DEV).to(dtype)
    gf, gb, dz = vm.vm_pool_scan_repeat_bwd(fwd, dout, bwd=bwd, z=z, pool_axis=0)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.pool_scan_repeat_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                                 pool_axis=0)
    for got, want, tag in ((gf, wf, "fwd"), (gb, wb, "bwd")):
        for k in _GRAD_KEYS:
            assert_close(host(got[k]), want[k], FP32_TOL, f"{tag} d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


# ---------------------------------------------------------------- full-size workloads
def test_full_vim_tiny_bidir():
    w = wl.WORKLOADS[1]
    _case(f"full {w.name}")
    fwd, bwd, z = wl.bidir_inputs(1001, w.batch, w.dim, w.seqlen, device=DEV, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    bsel = [0, 1, 31, 64, 100, 127]
    dsel = list(range(w.dim))
    ref = oracle.bidir_scan(sub_dir(host_dir(fwd), bsel, dsel), sub_dir(host_dir(bwd), bsel, dsel),
                            z=host(z)[bsel][:, dsel], combine_scale=w.combine_scale)
    assert_close(host(out[bsel]), ref, FP32_TOL, "vim-t full (sampled batches)")


@pytest.mark.parametrize("bidir", [False, True])
def test_long_sequence(bidir):
    # 2^20 steps (the offsets stay far from the 2 GiB resource limit, which
    # the host rejects before launch): every element, against the oracle
    L = 1 << 20
    _case(f"long sequence L={L} bidir={bidir}")
    if bidir:
        fwd, bwd, z = wl.bidir_inputs(1300, 1, 16, L, device=DEV, perturb=True)
        out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
        torch.cuda.synchronize()
        ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z))
    else:
        p, z = wl.single_inputs(1301, 1, 16, L, device=DEV)
        out = vm.vm_selective_scan_fwd(**p, z=z, reverse=True)
        torch.cuda.synchronize()
        ref = oracle.selective_scan(**host_dir(p), z=host(z), reverse=True)
    assert_close(host(out), ref, FP32_TOL, "long")


def test_full_single():
    w = wl.WORKLOADS[0]
    _case(f"full {w.name}")
    p, z = wl.single_inputs(1000, w.batch, w.dim, w.seqlen, device=DEV)
    out = vm.vm_selective_scan_fwd(**p, z=z)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z))
    assert_close(host(out), ref, FP32_TOL, "single full")


def test_full_vim_small_bf16():
    w = wl.WORKLOADS[2]
    _case(f"full {w.name}")
    fwd, bwd, z = wl.bidir_inputs(1002, w.batch, w.dim, w.seqlen, device=DEV,
                                  dtype=torch.bfloat16, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    torch.cuda.synchronize()
    bsel = [0, 15]
    dsel = list(range(0, w.dim, 7)) + [w.dim - 1]
    hf, hb = host_dir(fwd), host_dir(bwd)
    ref = oracle.bidir_scan(sub_dir(hf, bsel, dsel), sub_dir(hb, bsel, dsel), z=host(z)[bsel][:, dsel])
    assert_close(host(out)[bsel][:, dsel], ref, BF16_TOL, "vim-s bf16 full (sampled)")


@pytest.mark.parametrize("size", [56, 57])
def test_full_es2d(size):
    w = wl.WORKLOADS[3]
    _case(f"full {w.name} {size}")
    x, p = wl.es2d_inputs(1003 + size, w.batch, w.dim, size, size, device=DEV)
    s = vm.vm_atrous_gather(x)
    Lg = s.shape[-1]
    y = vm.vm_selective_scan_fwd(s.reshape(4 * w.batch, w.dim, Lg), **p)
    out = vm.vm_atrous_scatter(y.reshape(w.batch, 4, w.dim, Lg), size, size)
    torch.cuda.synchronize()
    # gather / scatter bit-exact over the whole batch
    assert np.array_equal(host(s), oracle.atrous_gather(host(x)))
    bsel = [0, 37, 63]
    rows = [4 * b + k for b in bsel for k in range(4)]
    hp = host_dir(p)
    hs = oracle.atrous_gather(host(x)[bsel])
    hy = oracle.selective_scan(hs.reshape(4 * len(bsel), w.dim, Lg),
                               hp["delta"][rows], hp["A"], hp["B"][rows], hp["C"][rows], hp["D"],
                               delta_bias=hp["delta_bias"])
    ref = oracle.atrous_scatter(hy.reshape(len(bsel), 4, w.dim, Lg), size, size)
    assert_close(host(out)[bsel], ref, FP32_TOL, f"es2d full {size}")


@pytest.mark.parametrize("axis", [0, 1])
def test_full_fastvim_pooled(axis):
    w = wl.WORKLOADS[4]
    _case(f"full {w.name} pooled axis{axis}")
    fwd, bwd, z = wl.fastvim_inputs(1004, w.batch, w.dim, w.height, w.width, axis, device=DEV)
    out = vm.vm_pool_scan_repeat(fwd, bwd, z=z, combine_scale=w.combine_scale, pool_axis=axis)
    torch.cuda.synchronize()
    bsel, dsel = [0, 127], [0, 1, 190, 383]
    hf = {k: host(v[bsel][:, dsel]) if k in ("u", "delta") else None for k, v in fwd.items()}
    hb = {k: host(v[bsel][:, dsel]) if k in ("u", "delta") else None for k, v in bwd.items()}
    for h, p in ((hf, fwd), (hb, bwd)):
        h["A"], h["D"], h["delta_bias"] = host(p["A"])[dsel], host(p["D"])[dsel], host(p["delta_bias"])[dsel]
        h["B"], h["C"] = host(p["B"][bsel]), host(p["C"][bsel])
    ref = oracle.pool_scan_repeat(hf, hb, z=host(z[bsel][:, dsel]), combine_scale=w.combine_scale,
                                  pool_axis=axis)
    assert_close(host(out[bsel][:, dsel]), ref, FP32_TOL, f"fastvim pooled axis{axis}")


def test_full_fastvim_unpooled():
    w = wl.WORKLOADS[4]
    _case(f"full {w.name} unpooled L={w.height * w.width}")
    fwd, bwd, z = wl.fastvim_inputs(1004, w.batch, w.dim, w.height, w.width, 0, device=DEV,
                                    full_resolution=True)
    L = w.height * w.width
    for p in (fwd, bwd):
        p["u"] = p["u"].reshape(w.batch, w.dim, L)
    zf = z.reshape(w.batch, w.dim, L)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=zf, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    bsel, dsel = [5, 120], [0, 100, 383]
    ref = oracle.bidir_scan(sub_dir({k: host(v[bsel]) if k in ("u", "delta", "B", "C") else host(v)
                                     for k, v in fwd.items()}, list(range(2)), dsel),
                            sub_dir({k: host(v[bsel]) if k in ("u", "delta", "B", "C") else host(v)
                                     for k, v in bwd.items()}, list(range(2)), dsel),
                            z=host(zf[bsel][:, dsel]), combine_scale=w.combine_scale)
    assert_close(host(out[bsel][:, dsel]), ref, FP32_TOL, "fastvim unpooled (sampled)")


# ---------------------------------------------------------------- SS2D
def _ss2d_ref(u, dirs, z, scale=1.0, softplus=True, bsel=None, dsel=None):
    hu, hz = host(u), host(z)
    hd = [host_dir(p) for p in dirs]
    if bsel is not None:
        hu, hz = hu[bsel][:, dsel], (hz[bsel][:, dsel] if hz is not None else None)
        hd = [sub_dir(p, bsel, dsel) for p in hd]
    return oracle.ss2d_scan(hu, hd, z=hz, combine_scale=scale, delta_softplus=softplus)


# (1, 1) degenerate map; (3, 5) and (33, 17) ragged 32 x 32 transpose tiles;
# (7, 10) single tile; (12, 32) wide rows; (20, 32) and (24, 25): 640 and 600
# steps, past the on-chip exchange (line-aligned and ragged global exchange).
# (12, 32), (20, 32), (68, 8): four-wide transpose and merge.
@pytest.mark.parametrize("H,W", [(1, 1), (3, 5), (7, 10), (12, 32), (33, 17), (20, 32), (24, 25),
                                 (68, 8)])
@pytest.mark.parametrize("bc_layout", ["token", "dense"])
def test_ss2d_fp32(H, W, bc_layout):
    _case(f"ss2d fp32 {H}x{W} bc {bc_layout}")
    u, dirs, z = wl.ss2d_inputs(800 + H * W, 2, 70, H, W, device=DEV, perturb=True, bc_layout=bc_layout)
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    assert_close(host(out), _ss2d_ref(u, dirs, z, 0.5), FP32_TOL, f"ss2d {H}x{W}")


def test_ss2d_ungated_no_softplus():
    _case("ss2d ungated no softplus 9x6")
    u, dirs, _ = wl.ss2d_inputs(850, 2, 33, 9, 6, dstate=7, device=DEV, gated=False, perturb=True)
    for p in dirs:
        p["delta"] = torch.rand_like(p["delta"]) * 0.2
        p["delta_bias"] = None
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=None, combine_scale=1.0, delta_softplus=False)
    torch.cuda.synchronize()
    ref = _ss2d_ref(u, dirs, None, 1.0, softplus=False)
    assert_close(host(out), ref, FP32_TOL, "ss2d ungated")


# 13 x 37: scalar transpose and merge; 68 x 132: the four-wide 64 x 64 tiles
# with ragged edges in both directions
@pytest.mark.parametrize("H,W", [(13, 37), (68, 132)])
def test_ss2d_column_routing_bit_exact(H, W):
    # B = 0 and D_k = 1: every traversal returns u at its own pixel, so the
    # merged output is exactly 4u (any misrouted pixel breaks equality)
    _case(f"ss2d routing bit-exact {H}x{W}")
    u, dirs, _ = wl.ss2d_inputs(860, 2, 5, H, W, device=DEV, gated=False)
    for p in dirs:
        p["B"] = torch.zeros_like(p["B"])
        p["D"] = torch.ones_like(p["D"])
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=None)
    torch.cuda.synchronize()
    assert bits_equal(out, _ss2d_ref(u, dirs, None))


@pytest.mark.parametrize("H,W", [(12, 10), (20, 32)])
def test_ss2d_bf16(H, W):
    _case(f"ss2d bf16 {H}x{W}")
    u, dirs, z = wl.ss2d_inputs(870 + H, 2, 70, H, W, device=DEV, dtype=torch.bfloat16)
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=z)
    torch.cuda.synchronize()
    assert_close(host(out), _ss2d_ref(u, dirs, z), BF16_TOL, "ss2d bf16")


def test_full_ss2d():
    w = wl.WORKLOADS[5]
    _case(f"full {w.name}")
    u, dirs, z = wl.ss2d_inputs(1005, w.batch, w.dim, w.height, w.width, device=DEV, perturb=True)
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=z, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    bsel, dsel = [0, 63], [0, 17, 100, 191]
    ref = _ss2d_ref(u, dirs, z, w.combine_scale, bsel=bsel, dsel=dsel)
    assert_close(host(out)[bsel][:, dsel], ref, FP32_TOL, "ss2d full (sampled)")


# ---------------------------------------------------------------- zero-order hold
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("L", [77, 600])
def test_zoh_single_fp32(reverse, L):
    _case(f"zoh single fp32 L{L} rev{reverse}")
    p, z = wl.single_inputs(1500 + L, 2, 70, L, device=DEV, perturb=True)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse, zoh=True)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), reverse=reverse, zoh=True)
    assert_close(host(out), ref, FP32_TOL, "zoh single")


def test_zoh_branch_boundary():
    # dt A spread over [-0.6, -0.002] without softplus: both sides of the
    # |dt A| = 1/8 switch between the series and exp(dt A) - 1, plus A = 0
    # states (dstate 5 of 16 lanes' worth: padded states too)
    _case("zoh branch boundary")
    p, z = wl.single_inputs(1510, 2, 40, 64, dstate=5, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(1511)
    p["delta"] = 0.01 + 0.3 * torch.rand(p["delta"].shape, generator=g, device=DEV)
    p["delta_bias"] = None
    p["A"] = -(0.2 + 1.8 * torch.rand(p["A"].shape, generator=g, device=DEV))
    p["A"][:, 0] = 0.0
    out = vm.vm_selective_scan_fwd(**p, z=z, delta_softplus=False, zoh=True)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**host_dir(p), z=host(z), delta_softplus=False, zoh=True)
    assert_close(host(out), ref, FP32_TOL, "zoh boundary")


@pytest.mark.parametrize("L", [197, 600])
def test_zoh_bidir_fp32(L):
    _case(f"zoh bidir fp32 L{L}")
    fwd, bwd, z = wl.bidir_inputs(1520 + L, 2, 70, L, device=DEV, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5, zoh=True)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z), combine_scale=0.5, zoh=True)
    assert_close(host(out), ref, FP32_TOL, "zoh bidir")


def test_zoh_bidir_bf16():
    _case("zoh bidir bf16 L333")
    fwd, bwd, z = wl.bidir_inputs(1530, 2, 70, 333, device=DEV, dtype=torch.bfloat16)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, zoh=True)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(z), zoh=True)
    assert_close(host(out), ref, BF16_TOL, "zoh bidir bf16")


def test_zoh_pool_and_ss2d():
    _case("zoh pool 12x32 axis1 and ss2d 9x14")
    fwd, bwd, z = wl.fastvim_inputs(1540, 2, 70, 12, 32, 1, device=DEV, perturb=True)
    out = vm.vm_pool_scan_repeat(fwd, bwd, z=z, pool_axis=1, zoh=True)
    u, dirs, z2 = wl.ss2d_inputs(1541, 2, 70, 9, 14, device=DEV, perturb=True)
    out2 = vm.vm_ss2d_scan_fwd(u, dirs, z=z2, zoh=True)
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(bwd), z=host(z), pool_axis=1, zoh=True)
    assert_close(host(out), ref, FP32_TOL, "zoh pool")
    assert_close(host(out2), _ss2d_ref_zoh(u, dirs, z2), FP32_TOL, "zoh ss2d")


def _ss2d_ref_zoh(u, dirs, z):
    return oracle.ss2d_scan(host(u), [host_dir(p) for p in dirs], z=host(z), zoh=True)


def test_full_vim_tiny_bidir_zoh():
    w = wl.WORKLOADS[1]
    _case(f"full {w.name} zoh")
    fwd, bwd, z = wl.bidir_inputs(1550, w.batch, w.dim, w.seqlen, device=DEV, perturb=True)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=w.combine_scale, zoh=True)
    torch.cuda.synchronize()
    bsel, dsel = [0, 77, 127], list(range(w.dim))
    ref = oracle.bidir_scan(sub_dir(host_dir(fwd), bsel, dsel), sub_dir(host_dir(bwd), bsel, dsel),
                            z=host(z)[bsel][:, dsel], combine_scale=w.combine_scale, zoh=True)
    assert_close(host(out[bsel]), ref, FP32_TOL, "vim-t zoh full (sampled batches)")


# ---------------------------------------------------------------- causal conv1d + SiLU
def _conv_inputs(seed, batch, dim, L, dtype=torch.float32):
    g = wl.generator(seed, DEV)
    x = torch.randn((batch, dim, L), generator=g, device=DEV).to(dtype)
    w, b = wl.conv_params(g, dim, DEV)
    return x, w, b


# L = 2: shorter than the kernel; 2500: three 1024-step chunks (margins
# across chunk boundaries); 197: one ragged chunk
@pytest.mark.parametrize("batch,dim,L", [(2, 70, 197), (1, 3, 2500), (2, 5, 2)])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv1d_silu(batch, dim, L, reverse, dtype):
    _case(f"conv1d b{batch} d{dim} L{L} rev{reverse} {dtype}")
    x, w, b = _conv_inputs(1600 + L, batch, dim, L, dtype)
    out = vm.vm_causal_conv1d_silu(x, w, b, reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.causal_conv1d_silu(host(x), host(w), host(b), reverse=reverse)
    if dtype == torch.float32:
        assert_close(host(out), ref, FP32_TOL, "conv1d")
    else:   # one bf16 rounding of the result: within 2^-8 relative per element
        assert np.all(np.abs(host(out) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("L,reverse", [(77, False), (77, True), (300, True), (16, False), (3, True)])
@pytest.mark.parametrize("zoh", [False, True])
def test_fused_conv_single(L, reverse, zoh):
    _case(f"fused conv single L{L} rev{reverse} zoh{zoh}")
    p, z = wl.single_inputs(1700 + L, 2, 70, L, device=DEV, perturb=True)
    g = wl.generator(1800 + L, DEV)
    cw, cb = wl.conv_params(g, 70, DEV)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse, zoh=zoh, conv_w=cw, conv_b=cb)
    torch.cuda.synchronize()
    hp = host_dir(p)
    hp["u"] = oracle.causal_conv1d_silu(hp["u"], host(cw), host(cb), reverse=reverse)
    ref = oracle.selective_scan(**hp, z=host(z), reverse=reverse, zoh=zoh)
    assert_close(host(out), ref, FP32_TOL, "fused conv single")


# 520 / 521: the last on-chip-exchange length with the conv rows in LDS, and
# the first global one
@pytest.mark.parametrize("L", [197, 520, 521, 600])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("zoh", [False, True])
def test_fused_conv_bidir(L, dtype, zoh):
    # both directions read the same content x through their own convolutions:
    # the backward one runs on the reversed sequence; with zoh the write is
    # the zero-order-hold coefficient ("Norm or Direction?" page, section 3,
    # eq. 2) on both sides of the on-chip / global exchange boundary
    _case(f"fused conv bidir L{L} {dtype} zoh{zoh}")
    fwd, bwd, z = wl.bidir_inputs(1900 + L, 2, 70, L, device=DEV, dtype=dtype, perturb=True)
    bwd["u"] = fwd["u"]
    g = wl.generator(2000 + L, DEV)
    for p in (fwd, bwd):
        p["conv_w"], p["conv_b"] = wl.conv_params(g, 70, DEV)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5, zoh=zoh)
    torch.cuda.synchronize()
    hf, hb = host_dir(fwd), host_dir(bwd)
    for h, rev in ((hf, False), (hb, True)):
        h["u"] = oracle.causal_conv1d_silu(h["u"], h.pop("conv_w"), h.pop("conv_b"), reverse=rev)
    ref = oracle.bidir_scan(hf, hb, z=host(z), combine_scale=0.5, zoh=zoh)
    assert_close(host(out), ref, FP32_TOL if dtype == torch.float32 else BF16_TOL, "fused conv bidir")


# The global exchange splits a channel's 16 states over 8 lanes (two states
# each, B and C read per lane) when a 4-lane split would leave fewer than two
# waves per SIMD: 2 x 44 channels (dim 44 = 5 x 8 + 4, a partial last row
# block) take the 8-lane split, 64 x 256 (2048 waves) the 4-lane one.  Every
# write option on both.
@pytest.mark.parametrize("batch,dim", [(2, 44), (64, 256)])
@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("conv", [False, True])
def test_bidir_global_exchange_state_splits(batch, dim, zoh, conv):
    L = 600
    _case(f"bidir global exchange b{batch} d{dim} zoh{zoh} conv{conv}")
    fwd, bwd, z = wl.bidir_inputs(2100 + dim, batch, dim, L, device=DEV, perturb=True)
    if conv:
        bwd["u"] = fwd["u"]
        g = wl.generator(2200 + dim, DEV)
        for p in (fwd, bwd):
            p["conv_w"], p["conv_b"] = wl.conv_params(g, dim, DEV)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5, zoh=zoh)
    torch.cuda.synchronize()
    hf, hb = host_dir(fwd), host_dir(bwd)
    if conv:
        for h, rev in ((hf, False), (hb, True)):
            h["u"] = oracle.causal_conv1d_silu(h["u"], h.pop("conv_w"), h.pop("conv_b"), reverse=rev)
    ref = oracle.bidir_scan(hf, hb, z=host(z), combine_scale=0.5, zoh=zoh)
    assert_close(host(out), ref, FP32_TOL, "global exchange state split")


def test_full_vim_tiny_bidir_fused_conv():
    """The Vim-T block with its causal conv1d + SiLU inside the scan, at full
    size (two row blocks per workgroup): sampled batch rows against the
    oracle, and every element bit-equal to the conv kernels then the scan."""
    w = wl.WORKLOADS[1]
    _case(f"full {w.name} fused conv")
    fwd, bwd, z = wl.bidir_inputs(1002, w.batch, w.dim, w.seqlen, device=DEV, perturb=True)
    bwd["u"] = fwd["u"]
    g = wl.generator(1003, DEV)
    for p in (fwd, bwd):
        p["conv_w"], p["conv_b"] = wl.conv_params(g, w.dim, DEV)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=w.combine_scale)
    f2 = {k: v for k, v in fwd.items() if not k.startswith("conv")}
    b2 = {k: v for k, v in bwd.items() if not k.startswith("conv")}
    f2["u"] = vm.vm_causal_conv1d_silu(fwd["u"], fwd["conv_w"], fwd["conv_b"])
    b2["u"] = vm.vm_causal_conv1d_silu(bwd["u"], bwd["conv_w"], bwd["conv_b"], reverse=True)
    two = vm.vm_bidir_scan_fwd(f2, b2, z=z, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    bsel = [0, 63, 127]
    dsel = list(range(w.dim))
    hf, hb = sub_dir(host_dir(fwd), bsel, dsel), sub_dir(host_dir(bwd), bsel, dsel)
    for h, rev in ((hf, False), (hb, True)):
        h["u"] = oracle.causal_conv1d_silu(h["u"], h.pop("conv_w"), h.pop("conv_b"), reverse=rev)
    ref = oracle.bidir_scan(hf, hb, z=host(z)[bsel][:, dsel], combine_scale=w.combine_scale)
    assert_close(host(out[bsel]), ref, FP32_TOL, "vim-t fused conv full (sampled batches)")


@pytest.mark.parametrize("L", [1, 2, 3, 9, 197])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv1d_silu_bwd(L, reverse, dtype):
    _case(f"conv bwd L{L} rev{reverse} {dtype}")
    g = wl.generator(3200 + L, DEV)
    x = torch.randn((3, 70, L), generator=g, device=DEV).to(dtype)
    w, b = wl.conv_params(g, 70, DEV)
    du = torch.randn((3, 70, L), generator=g, device=DEV)
    dx, dw, db = vm.vm_causal_conv1d_silu_bwd(x, w, du, bias=b, reverse=reverse)
    torch.cuda.synchronize()
    wx, ww, wb, _ = ograd.causal_conv1d_silu_grad(host(x), host(w), host(b), host(du), reverse=reverse)
    assert_close(host(dx), wx, FP32_TOL, "dx")
    assert_close(host(dw), ww, FP32_TOL, "dw")
    assert_close(host(db), wb, FP32_TOL, "dbias")


def test_conv1d_silu_bwd_chunks_and_no_bias():
    """Many batch rows per channel (several chunks per channel), no bias:
    dbias of the zero bias is still the sum of dv; deterministic."""
    _case("conv bwd chunks, no bias")
    g = wl.generator(3300, DEV)
    x = torch.randn((300, 24, 50), generator=g, device=DEV)
    w, _ = wl.conv_params(g, 24, DEV)
    du = torch.randn(x.shape, generator=g, device=DEV)
    dx, dw, db = vm.vm_causal_conv1d_silu_bwd(x, w, du, with_dbias=True)
    dx2, dw2, db2 = vm.vm_causal_conv1d_silu_bwd(x, w, du, with_dbias=True)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2) and torch.equal(db, db2)
    wx, ww, _, _ = ograd.causal_conv1d_silu_grad(host(x), host(w), None, host(du))
    zb = np.zeros(24)
    _, _, wb, _ = ograd.causal_conv1d_silu_grad(host(x), host(w), zb, host(du))
    assert_close(host(dx), wx, FP32_TOL, "dx")
    assert_close(host(dw), ww, FP32_TOL, "dw")
    assert_close(host(db), wb, FP32_TOL, "dbias")
    _, _, none = vm.vm_causal_conv1d_silu_bwd(x, w, du)
    assert none is None


def test_conv_and_scan_backward_chain():
    """Training a Vim branch: the scan backward's du feeds the conv backward,
    against the oracle's chained gradients."""
    _case("conv + scan backward chain")
    p, z = wl.single_inputs(3400, 2, 40, 60, device=DEV, gated=True, perturb=True)
    g = wl.generator(3401, DEV)
    x = p["u"].clone()
    w, b = wl.conv_params(g, 40, DEV)
    p["u"] = vm.vm_causal_conv1d_silu(x, w, b)
    dout = torch.randn(x.shape, generator=g, device=DEV)
    gs, _ = vm.vm_selective_scan_bwd(p, dout, z=z)
    dx, dw, db = vm.vm_causal_conv1d_silu_bwd(x, w, gs["u"], bias=b)
    torch.cuda.synchronize()
    hp = host_dir(p)
    hp["u"] = oracle.causal_conv1d_silu(host(x), host(w), host(b))
    want, _, _ = ograd.selective_scan_grad(hp, host(dout), z=host(z))
    wx, ww, wb, _ = ograd.causal_conv1d_silu_grad(host(x), host(w), host(b), want["u"])
    assert_close(host(dx), wx, FP32_TOL, "dx")
    assert_close(host(dw), ww, FP32_TOL, "dw")
    assert_close(host(db), wb, FP32_TOL, "dbias")


@pytest.mark.parametrize("L", [197, 600])
def test_fused_conv_equals_conv_then_scan(L):
    # the in-kernel convolution takes the same fp32 operations in the same
    # order as the standalone kernel, so both routes agree bit for bit
    _case(f"fused conv == conv then scan L{L}")
    fwd, bwd, z = wl.bidir_inputs(2100 + L, 2, 70, L, device=DEV, perturb=True)
    bwd["u"] = fwd["u"]
    g = wl.generator(2200 + L, DEV)
    for p in (fwd, bwd):
        p["conv_w"], p["conv_b"] = wl.conv_params(g, 70, DEV)
    fused = vm.vm_bidir_scan_fwd(fwd, bwd, z=z)
    f2 = {k: v for k, v in fwd.items() if not k.startswith("conv")}
    b2 = {k: v for k, v in bwd.items() if not k.startswith("conv")}
    f2["u"] = vm.vm_causal_conv1d_silu(fwd["u"], fwd["conv_w"], fwd["conv_b"])
    b2["u"] = vm.vm_causal_conv1d_silu(bwd["u"], bwd["conv_w"], bwd["conv_b"], reverse=True)
    two = vm.vm_bidir_scan_fwd(f2, b2, z=z)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)


# ---------------------------------------------------------------- HIP graph replay
def test_graph_replay_matches_eager():
    # the benchmark replays captured steps: every replay, with eager work and
    # synchronisations between replays, must equal the eager result exactly
    _case("graph replay: bidir L197 + ES2D 13x10")
    fwd, bwd, z = wl.bidir_inputs(2300, 4, 64, 197, device=DEV, perturb=True)
    x, p = wl.es2d_inputs(2301, 2, 32, 13, 10, device=DEV)
    Lg = vm.vm_atrous_group_len(13, 10)
    out = torch.empty_like(fwd["u"])
    s = torch.empty((2, 4, 32, Lg), device=DEV)
    y = torch.empty((8, 32, Lg), device=DEV)
    y2 = torch.empty((2, 32, 13, 10), device=DEV)

    def step():
        vm.vm_bidir_scan_fwd(fwd, bwd, z=z, out=out)
        vm.vm_atrous_gather(x, out=s)
        vm.vm_selective_scan_fwd(s.view(8, 32, Lg), **p, out=y)
        vm.vm_atrous_scatter(y.view(2, 4, 32, Lg), 13, 10, out=y2)

    step()
    torch.cuda.synchronize()
    want = (out.clone(), y2.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = wl.bidir_inputs(2302, 4, 64, 197, device=DEV)
    for r in range(3):
        out.fill_(float("nan"))
        y2.fill_(float("nan"))
        vm.vm_bidir_scan_fwd(other[0], other[1], z=other[2])      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]), f"replay {r}: bidir differs"
        assert torch.equal(y2, want[1]), f"replay {r}: ES2D differs"


# ---------------------------------------------------------------- backward
from oracle import grad as ograd  # noqa: E402

_GRAD_KEYS = ("u", "delta", "A", "B", "C", "D", "delta_bias")


def _dense_bc(p):
    return {k: (v.contiguous() if k in ("B", "C") else v) for k, v in p.items()}


@pytest.mark.parametrize("L", [1, 8, 77, 197])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("gated", [True, False])
def test_bwd_single(L, reverse, gated):
    _case(f"bwd single L{L} rev{reverse} gated{gated}")
    p, z = wl.single_inputs(2500 + L, 2, 70, L, device=DEV, gated=gated, perturb=True)
    dout = torch.randn(p["u"].shape, generator=wl.generator(2600 + L, DEV), device=DEV)
    g, dz = vm.vm_selective_scan_bwd(p, dout, z=z, reverse=reverse)
    torch.cuda.synchronize()
    want, wdz, _ = ograd.selective_scan_grad(host_dir(p), host(dout), z=host(z), reverse=reverse)
    for k in _GRAD_KEYS:
        assert_close(host(g[k]), want[k], FP32_TOL, f"d{k}")
    if gated:
        assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("L", [1, 9, 77])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("gated", [False, True])
def test_bwd_zoh_single(L, reverse, gated):
    """Zero-order-hold write: steps on both sides of the coefficient's series
    switch, and one state with A = 0 (coefficient dt)."""
    _case(f"bwd zoh single L{L} rev{reverse} gated{gated}")
    p, z = wl.single_inputs(2800 + L, 2, 70, L, device=DEV, gated=gated, perturb=True)
    p["A"][:, 3] = 0.0
    dout = torch.randn(p["u"].shape, generator=wl.generator(2900 + L, DEV), device=DEV)
    g, dz = vm.vm_selective_scan_bwd(p, dout, z=z, reverse=reverse, zoh=True)
    torch.cuda.synchronize()
    want, wdz, _ = ograd.selective_scan_grad(host_dir(p), host(dout), z=host(z), reverse=reverse,
                                             zoh=True)
    for k in _GRAD_KEYS:
        assert_close(host(g[k]), want[k], FP32_TOL, f"d{k}")
    if gated:
        assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("L", [77, 600])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bwd_zoh_bidir(L, dtype):
    _case(f"bwd zoh bidir L{L} {dtype}")
    fwd, bwd, z = wl.bidir_inputs(3000 + L, 2, 40, L, device=DEV, dtype=dtype, perturb=True)
    dout = torch.randn(z.shape, generator=wl.generator(3100 + L, DEV), device=DEV).to(dtype)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5, zoh=True)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=0.5, zoh=True)
    tol = FP32_TOL          # bf16 inputs are widened exactly; the oracle sees the same values
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], tol, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], tol, f"bwd d{k}")
    assert_close(host(dz), wdz, tol, "dz")


def _conv_scan_inputs(p):
    """Host copy of a conv direction with u replaced by the oracle's conv output."""
    h = host_dir(p)
    x, w, b = h.pop("u"), h.pop("conv_w"), h.pop("conv_b", None)
    return h, x, w, b


@pytest.mark.parametrize("L", [77, 600])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("zoh", [False, True])
def test_bwd_bidir_fused_conv(L, dtype, zoh):
    """Backward of the bidirectional scan with the fused conv (both
    directions reading the same x through their own convolutions), with
    either write."""
    _case(f"bwd bidir fused conv L{L} {dtype} zoh{zoh}")
    fwd, bwd, z = wl.bidir_inputs(3500 + L, 2, 40, L, device=DEV, dtype=dtype, perturb=True)
    bwd["u"] = fwd["u"]
    g = wl.generator(3600 + L, DEV)
    for q in (fwd, bwd):
        q["conv_w"], q["conv_b"] = wl.conv_params(g, 40, DEV)
    dout = torch.randn(z.shape, generator=g, device=DEV).to(dtype)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5, zoh=zoh)
    torch.cuda.synchronize()
    hf, xf, wf_, bf_ = _conv_scan_inputs(fwd)
    hb, xb, wb_, bb_ = _conv_scan_inputs(bwd)
    hf["u"] = oracle.causal_conv1d_silu(xf, wf_, bf_)
    hb["u"] = oracle.causal_conv1d_silu(xb, wb_, bb_, reverse=True)
    wantf, wantb, wdz, _ = ograd.bidir_scan_grad(hf, hb, host(dout), z=host(z), combine_scale=0.5, zoh=zoh)
    for got, want, x, w, b, rev, tag in ((gf, wantf, xf, wf_, bf_, False, "fwd"),
                                         (gb, wantb, xb, wb_, bb_, True, "bwd")):
        dx, dw, db, _ = ograd.causal_conv1d_silu_grad(x, w, b, want["u"], reverse=rev)
        assert_close(host(got["u"]), dx, FP32_TOL, f"{tag} dx")
        assert_close(host(got["conv_w"]), dw, FP32_TOL, f"{tag} dconv_w")
        assert_close(host(got["conv_b"]), db, FP32_TOL, f"{tag} dconv_b")
        for k in _GRAD_KEYS[1:]:
            assert_close(host(got[k]), want[k], FP32_TOL, f"{tag} d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("zoh", [False, True])
def test_bwd_single_fused_conv(reverse, zoh):
    _case(f"bwd single fused conv rev{reverse} zoh{zoh}")
    p, z = wl.single_inputs(3700 + reverse, 2, 40, 50, device=DEV, gated=True, perturb=True)
    g = wl.generator(3710 + reverse, DEV)
    p["conv_w"], _ = wl.conv_params(g, 40, DEV)          # no conv bias
    dout = torch.randn(p["u"].shape, generator=g, device=DEV)
    got, dz = vm.vm_selective_scan_bwd(p, dout, z=z, reverse=reverse, zoh=zoh)
    torch.cuda.synchronize()
    assert got["conv_b"] is None
    h, x, w, _ = _conv_scan_inputs(p)
    h["u"] = oracle.causal_conv1d_silu(x, w, None, reverse=reverse)
    want, wdz, _ = ograd.selective_scan_grad(h, host(dout), z=host(z), reverse=reverse, zoh=zoh)
    dx, dw, _, _ = ograd.causal_conv1d_silu_grad(x, w, None, want["u"], reverse=reverse)
    assert_close(host(got["u"]), dx, FP32_TOL, "dx")
    assert_close(host(got["conv_w"]), dw, FP32_TOL, "dconv_w")
    for k in _GRAD_KEYS[1:]:
        assert_close(host(got[k]), want[k], FP32_TOL, f"d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("size", [56, 57])
def test_es2d_backward_by_composition(size):
    """ES2D gradients from the entry points: gather and scatter are each
    other's adjoints (pinned on the oracle), so the map gradient is
    scatter(scan backward(gather(dout))) and pads get none."""
    _case(f"es2d backward composition {size}")
    batch, ch, N = 2, 24, 16
    g = wl.generator(3800 + size, DEV)
    x = torch.randn((batch, ch, size, size), generator=g, device=DEV)
    Lg = vm.vm_atrous_group_len(size, size)
    p, _ = wl.single_inputs(3810 + size, 4 * batch, ch, Lg, device=DEV, gated=False)
    p["u"] = vm.vm_atrous_gather(x).view(4 * batch, ch, Lg)
    dout = torch.randn(x.shape, generator=g, device=DEV)
    dstreams = vm.vm_atrous_gather(dout).view(4 * batch, ch, Lg)
    gs, _ = vm.vm_selective_scan_bwd(p, dstreams)
    dx = vm.vm_atrous_scatter(gs["u"].view(batch, 4, ch, Lg), size, size)
    torch.cuda.synchronize()
    hp = host_dir(p)
    hp["u"] = oracle.atrous_gather(host(x)).reshape(4 * batch, ch, Lg)
    want, _, _ = ograd.selective_scan_grad(hp, oracle.atrous_gather(host(dout)).reshape(4 * batch, ch, Lg))
    assert_close(host(dx), oracle.atrous_scatter(want["u"].reshape(batch, 4, ch, Lg), size, size),
                 FP32_TOL, "dx")
    for k in _GRAD_KEYS[1:]:
        assert_close(host(gs[k]), want[k], FP32_TOL, f"d{k}")


def test_bwd_small_dstate_no_softplus_dense_bc():
    _case("bwd N5 no softplus dense B/C")
    p, z = wl.single_inputs(2700, 3, 33, 50, dstate=5, device=DEV, bc_layout="dense")
    p["delta"] = torch.rand_like(p["delta"]) * 0.3
    p["delta_bias"] = None
    dout = torch.randn(p["u"].shape, generator=wl.generator(2701, DEV), device=DEV)
    g, dz = vm.vm_selective_scan_bwd(p, dout, z=z, delta_softplus=False)
    torch.cuda.synchronize()
    hp = host_dir(p)
    want, wdz, _ = ograd.selective_scan_grad(hp, host(dout), z=host(z), delta_softplus=False)
    for k in _GRAD_KEYS[:-1]:
        assert_close(host(g[k]), want[k], FP32_TOL, f"d{k}")
    assert g["delta_bias"] is None
    assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("L", [77, 600])
def test_bwd_bidir(L):
    _case(f"bwd bidir L{L}")
    fwd, bwd, z = wl.bidir_inputs(2800 + L, 2, 40, L, device=DEV, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(2900 + L, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=0.5)
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


def test_bwd_bidir_two_row_blocks_per_workgroup():
    """The fused backward preparation in workgroups of two row blocks (83 x
    25 = 2075 row blocks: the last workgroup's second one is empty, and the
    last of each batch row has 13 channels), writing tile-major checkpoints
    and dy that the backward kernel reads."""
    _case("bwd bidir two row blocks per workgroup")
    fwd, bwd, z = wl.bidir_inputs(2950, 83, 397, 9, device=DEV, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(2951, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=0.5)
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


def test_bwd_bidir_tiled_dy_rows_past_dim_ignored():
    """The tile-major output gradient has slots for all 16 channels of a
    block; with 29 channels the last block's three spare slots are never
    written, and the backward must not read them.  A first call with 32
    channels and a NaN output gradient (the same workspace sizes) leaves NaN
    in the workspace the second call is likely to be given back; the second
    call's gradients must still match the oracle."""
    _case("bwd bidir tiled dy rows past dim")
    fwd, bwd, z = wl.bidir_inputs(2960, 3, 32, 40, device=DEV, perturb=True)
    dout = torch.full(fwd["u"].shape, float("nan"), device=DEV)
    vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5)
    fwd, bwd, z = wl.bidir_inputs(2961, 3, 29, 40, device=DEV, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(2962, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=0.5)
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("batch,dim", [(2, 44), (64, 256)])
@pytest.mark.parametrize("zoh", [False, True])
def test_bwd_bidir_global_exchange_checkpoints_from_forward(batch, dim, zoh):
    """Long sequences (the global exchange, 8-lane split at 2 x 44 channels,
    4-lane at 64 x 256): with z, the forward recomputation stores the
    backward's checkpoints (at visit positions 0 and 8 of its 16-step tiles);
    without z, the backward kernel runs its own first pass.  The gated call
    must match the ungated one on dout SiLU(z) (which differs only in the
    rounding of dy) in every gradient but dz; the oracle checks the gated
    small case directly in test_bwd_bidir."""
    _case(f"bwd bidir global exchange ck from forward b{batch} d{dim} zoh{zoh}")
    L = 600
    fwd, bwd, z = wl.bidir_inputs(3100 + dim, batch, dim, L, device=DEV, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(3200 + dim, DEV), device=DEV)
    gf, gb, _ = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5, zoh=zoh)
    d2 = (dout * torch.nn.functional.silu(z)).contiguous()
    hf, hb, _ = vm.vm_bidir_scan_bwd(fwd, bwd, d2, z=None, combine_scale=0.5, zoh=zoh)
    torch.cuda.synchronize()
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), host(hf[k]), FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), host(hb[k]), FP32_TOL, f"bwd d{k}")


def test_bwd_bf16():
    # bf16 inputs: the pass runs in fp32 on their exact widening, so the
    # gradients match the oracle's (on the same bf16 values) to fp32 accuracy
    _case("bwd bf16 bidir L150")
    fwd, bwd, z = wl.bidir_inputs(3050, 2, 40, 150, device=DEV, dtype=torch.bfloat16, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(3051, DEV), device=DEV).to(torch.bfloat16)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z)
    torch.cuda.synchronize()
    assert gf["u"].dtype == torch.float32 and dz.dtype == torch.float32
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z))
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


def test_bwd_deterministic():
    _case("bwd deterministic")
    fwd, bwd, z = wl.bidir_inputs(3000, 4, 64, 100, device=DEV)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(3001, DEV), device=DEV)
    a = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z)
    b = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z)
    torch.cuda.synchronize()
    for ga, gb_ in ((a[0], b[0]), (a[1], b[1])):
        for k in _GRAD_KEYS:
            assert torch.equal(ga[k], gb_[k]), k
    assert torch.equal(a[2], b[2])


def test_full_vim_tiny_bidir_bwd():
    # the headline workload's backward, every gradient element
    w = wl.WORKLOADS[1]
    _case(f"full {w.name} backward")
    fwd, bwd, z = wl.bidir_inputs(3100, w.batch, w.dim, w.seqlen, device=DEV, perturb=True)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(3101, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=w.combine_scale)
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")


def _ss2d_bwd_check(u, dirs, dout, z, tag, scale=1.0, softplus=True, zoh=False):
    du, grads, dz = vm.vm_ss2d_scan_bwd(u, dirs, dout, z=z, combine_scale=scale, delta_softplus=softplus,
                                        zoh=zoh)
    torch.cuda.synchronize()
    wdu, wg, wdz, _ = ograd.ss2d_scan_grad(host(u), [host_dir(p) for p in dirs], host(dout), z=host(z),
                                           combine_scale=scale, delta_softplus=softplus, zoh=zoh)
    assert_close(host(du), wdu, FP32_TOL, f"{tag} du")
    for k in range(4):
        assert "u" not in grads[k]
        for key in _GRAD_KEYS[1:]:
            if wg[k][key] is None:
                assert grads[k][key] is None
            else:
                assert_close(host(grads[k][key]), wg[k][key], FP32_TOL, f"{tag} dir{k} d{key}")
    if z is None:
        assert dz is None
    else:
        assert_close(host(dz), wdz, FP32_TOL, f"{tag} dz")


@pytest.mark.parametrize("H,W,gated,bc_layout", [(5, 7, True, "token"), (8, 8, False, "token"),
                                                 (6, 9, True, "dense"), (24, 25, True, "token")])
def test_ss2d_bwd(H, W, gated, bc_layout):
    """Every gradient of the four-direction 2-D scan, against the oracle's
    autograd; 24 x 25 = 600 steps is past the on-chip exchange length."""
    _case(f"ss2d bwd {H}x{W} gated{gated} bc {bc_layout}")
    u, dirs, z = wl.ss2d_inputs(4200 + H * W, 2, 40, H, W, device=DEV, gated=gated, perturb=True,
                                bc_layout=bc_layout)
    dout = torch.randn(u.shape, generator=wl.generator(4201 + H, DEV), device=DEV)
    _ss2d_bwd_check(u, dirs, dout, z, f"ss2d bwd {H}x{W}", scale=0.5)


def test_ss2d_bwd_small_dstate_no_softplus():
    _case("ss2d bwd N7 no softplus 9x6")
    u, dirs, z = wl.ss2d_inputs(4300, 2, 33, 9, 6, dstate=7, device=DEV, perturb=True)
    g = wl.generator(4302, DEV)
    for k, p in enumerate(dirs):
        # without softplus the step is delta + bias as given: keep it positive
        p["delta"] = torch.rand(p["delta"].shape, generator=g, device=DEV) * 0.3
        p["delta_bias"] = None if k == 2 else torch.rand(p["D"].shape, generator=g, device=DEV) * 0.05
    dout = torch.randn(u.shape, generator=wl.generator(4301, DEV), device=DEV)
    _ss2d_bwd_check(u, dirs, dout, z, "ss2d bwd no softplus", softplus=False)


def test_ss2d_bwd_bf16_and_zoh():
    _case("ss2d bwd bf16 7x10, zoh 9x14")
    u, dirs, z = wl.ss2d_inputs(4400, 2, 40, 7, 10, device=DEV, dtype=torch.bfloat16, perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4401, DEV), device=DEV).to(torch.bfloat16)
    _ss2d_bwd_check(u, dirs, dout, z, "ss2d bwd bf16")
    u, dirs, z = wl.ss2d_inputs(4402, 2, 40, 9, 14, device=DEV, perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4403, DEV), device=DEV)
    _ss2d_bwd_check(u, dirs, dout, z, "ss2d bwd zoh", scale=0.5, zoh=True)


def test_ss2d_bwd_zoh_per_direction_launches():
    """SS2D backward with the zero-order-hold write where each traversal has
    at least 1024 row blocks (batch 64 x 16 blocks of 16 channels), so its
    four backward kernels launch one traversal at a time."""
    _case("ss2d bwd zoh b64 d256 3x4")
    u, dirs, z = wl.ss2d_inputs(4450, 64, 256, 3, 4, device=DEV, perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4451, DEV), device=DEV)
    _ss2d_bwd_check(u, dirs, dout, z, "ss2d bwd zoh per-direction", scale=0.5, zoh=True)


@pytest.mark.parametrize("H,W,dtype,gated,zoh", [(8, 12, torch.float32, True, False),
                                                  (12, 8, torch.bfloat16, True, False),
                                                  (4, 16, torch.float32, True, True),
                                                  (12, 4, torch.float32, False, False)])
def test_ss2d_bwd_four_wide_tiles(H, W, dtype, gated, zoh):
    """Maps with H and W multiples of 4 take the fused four-wide gate and
    map-gradient kernels (both layouts of the output gradient, the summed
    map gradient); the other SS2D backward cases take the separate ones."""
    _case(f"ss2d bwd four-wide {H}x{W} {dtype} gated{gated} zoh{zoh}")
    u, dirs, z = wl.ss2d_inputs(4460 + H * W, 2, 40, H, W, device=DEV, dtype=dtype, gated=gated,
                                perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4461 + H, DEV), device=DEV).to(dtype)
    _ss2d_bwd_check(u, dirs, dout, z, f"ss2d bwd four-wide {H}x{W}", scale=0.5, zoh=zoh)


def test_ss2d_bwd_four_wide_tiles_ragged():
    # 68 x 72: two 64 x 64 tiles per axis, the second one partial; sampled
    # (batch row, channel) pairs against the oracle
    _case("ss2d bwd four-wide 68x72 (sampled)")
    u, dirs, z = wl.ss2d_inputs(4470, 2, 40, 68, 72, device=DEV, perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4471, DEV), device=DEV)
    du, grads, dz = vm.vm_ss2d_scan_bwd(u, dirs, dout, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    bsel, dsel = [1], [0, 39]
    hd = [sub_dir(host_dir(p), bsel, dsel) for p in dirs]
    sel = lambda t: t[bsel][:, dsel]
    wdu, wg, wdz, _ = ograd.ss2d_scan_grad(sel(host(u)), hd, sel(host(dout)), z=sel(host(z)),
                                           combine_scale=0.5)
    assert_close(sel(host(du)), wdu, FP32_TOL, "ss2d 68x72 du (sampled)")
    assert_close(sel(host(dz)), wdz, FP32_TOL, "ss2d 68x72 dz (sampled)")
    for k in range(4):
        assert_close(sel(host(grads[k]["delta"])), wg[k]["delta"], FP32_TOL, f"ss2d 68x72 dir{k} ddelta")


def test_full_ss2d_bwd():
    # the full-size 2-D scan's backward; the map, delta and gate gradients of
    # sampled (batch row, channel) pairs depend on that pair's inputs only
    w = wl.WORKLOADS[5]
    _case(f"full {w.name} backward (sampled)")
    u, dirs, z = wl.ss2d_inputs(4500, w.batch, w.dim, w.height, w.width, device=DEV, perturb=True)
    dout = torch.randn(u.shape, generator=wl.generator(4501, DEV), device=DEV)
    du, grads, dz = vm.vm_ss2d_scan_bwd(u, dirs, dout, z=z, combine_scale=w.combine_scale)
    torch.cuda.synchronize()
    bsel, dsel = [0, w.batch - 1], [0, 17, w.dim - 1]
    hd = [sub_dir(host_dir(p), bsel, dsel) for p in dirs]
    sel = lambda t: t[bsel][:, dsel]
    wdu, wg, wdz, _ = ograd.ss2d_scan_grad(sel(host(u)), hd, sel(host(dout)), z=sel(host(z)),
                                           combine_scale=w.combine_scale)
    assert_close(sel(host(du)), wdu, FP32_TOL, "full ss2d du (sampled)")
    assert_close(sel(host(dz)), wdz, FP32_TOL, "full ss2d dz (sampled)")
    for k in range(4):
        assert_close(sel(host(grads[k]["delta"])), wg[k]["delta"], FP32_TOL, f"full ss2d dir{k} ddelta")


# ---------------------------------------------------------------- degenerate sizes
def test_degenerate_sizes_every_entry_point():
    # one channel, one batch row, shortest sequences / maps, for each entry
    _case("degenerate sizes")
    p, z = wl.single_inputs(3200, 1, 1, 1, dstate=1, device=DEV)
    out = vm.vm_selective_scan_fwd(**p, z=z)
    fwd, bwd, zb = wl.bidir_inputs(3201, 1, 1, 2, dstate=1, device=DEV)
    outb = vm.vm_bidir_scan_fwd(fwd, bwd, z=zb)
    u, dirs, z2 = wl.ss2d_inputs(3202, 1, 1, 1, 3, dstate=2, device=DEV)
    out2 = vm.vm_ss2d_scan_fwd(u, dirs, z=z2)
    x, w, b = _conv_inputs(3203, 1, 1, 1)
    outc = vm.vm_causal_conv1d_silu(x, w, b)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(3204, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=zb)
    torch.cuda.synchronize()
    assert_close(host(out), oracle.selective_scan(**host_dir(p), z=host(z)), FP32_TOL, "single 1x1x1")
    assert_close(host(outb), oracle.bidir_scan(host_dir(fwd), host_dir(bwd), z=host(zb)), FP32_TOL, "bidir L2")
    assert_close(host(out2), _ss2d_ref(u, dirs, z2), FP32_TOL, "ss2d 1x3")
    assert_close(host(outc), oracle.causal_conv1d_silu(host(x), host(w), host(b)), FP32_TOL, "conv L1")
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(zb))
    for k in _GRAD_KEYS:
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    assert_close(host(dz), wdz, FP32_TOL, "dz")
