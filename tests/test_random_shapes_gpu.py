"""Seeded random shapes and options through the C ABI against the oracles:
forward single and bidirectional scans, and the bidirectional backward; the
2-D paths (ES2D gather, group scan and scatter; SS2D forward and backward;
the FastVim pooled path forward and backward) on random maps.  The draws
cover the planner's branches (sequence-parallel single scan, 4- and 8-lane
splits, on-chip and global exchange, workgroups of one or two row blocks),
ragged tiles, partial row blocks, dstate below 16, both B/C layouts, the
zero-order-hold write, the fused conv, bf16 and the ungated scan; for the
maps, odd and even sides (the atrous padding) and sides that are and are not
multiples of 4 (the four-wide and the scalar layout kernels)."""
import random

import numpy as np
import pytest
import torch

import oracle
import selective_scan_fwd_amd as vm
from oracle import grad as ograd
from selective_scan_fwd_amd import workloads as wl

from _helpers import BF16_TOL, FP32_TOL, assert_close, host, host_dir

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
_GRAD_KEYS = ("u", "delta", "A", "B", "C", "D", "delta_bias")


def _draw(seed):
    r = random.Random(seed)
    L = r.choice([1, 7, 16, 33, 64, 100, 197, 256, 300, 553, 600, 700])
    batch = r.choice([1, 2, 3])
    dim = r.choice([1, 5, 16, 23, 40, 64, 97])
    dstate = r.choice([16, 16, 11, 4])
    return dict(L=L, batch=batch, dim=dim, dstate=dstate, zoh=r.random() < 0.3,
                conv=r.random() < 0.3, bf16=r.random() < 0.25, gated=r.random() < 0.8,
                reverse=r.random() < 0.5, bc_layout=r.choice(["token", "dense"]))


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _with_conv(p, g, dim):
    p["conv_w"], p["conv_b"] = wl.conv_params(g, dim, DEV)


def _host_conv(h, rev):
    h["u"] = oracle.causal_conv1d_silu(h["u"], h.pop("conv_w"), h.pop("conv_b"), reverse=rev)


@pytest.mark.parametrize("seed", range(12))
def test_random_single(seed):
    c = _draw(1000 + seed)
    _case(f"random single {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    p, z = wl.single_inputs(5000 + seed, c["batch"], c["dim"], c["L"], dstate=c["dstate"], device=DEV,
                            dtype=dt, gated=c["gated"], perturb=True, bc_layout=c["bc_layout"])
    if c["conv"]:
        _with_conv(p, wl.generator(5100 + seed, DEV), c["dim"])
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=c["reverse"], zoh=c["zoh"])
    torch.cuda.synchronize()
    h = host_dir(p)
    if c["conv"]:
        _host_conv(h, c["reverse"])
    ref = oracle.selective_scan(**h, z=host(z), reverse=c["reverse"], zoh=c["zoh"])
    assert_close(host(out), ref, BF16_TOL if c["bf16"] else FP32_TOL, "random single")


@pytest.mark.parametrize("seed", range(12))
def test_random_bidir(seed):
    c = _draw(2000 + seed)
    _case(f"random bidir {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    fwd, bwd, z = wl.bidir_inputs(6000 + seed, c["batch"], c["dim"], c["L"], dstate=c["dstate"], device=DEV,
                                  dtype=dt, gated=c["gated"], perturb=True, bc_layout=c["bc_layout"])
    if c["conv"]:
        bwd["u"] = fwd["u"]
        g = wl.generator(6100 + seed, DEV)
        _with_conv(fwd, g, c["dim"])
        _with_conv(bwd, g, c["dim"])
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5, zoh=c["zoh"])
    torch.cuda.synchronize()
    hf, hb = host_dir(fwd), host_dir(bwd)
    if c["conv"]:
        _host_conv(hf, False)
        _host_conv(hb, True)
    ref = oracle.bidir_scan(hf, hb, z=host(z), combine_scale=0.5, zoh=c["zoh"])
    assert_close(host(out), ref, BF16_TOL if c["bf16"] else FP32_TOL, "random bidir")


@pytest.mark.parametrize("seed", range(8))
def test_random_bidir_bwd(seed):
    c = _draw(3000 + seed)
    c["bf16"] = False
    _case(f"random bidir bwd {c}")
    fwd, bwd, z = wl.bidir_inputs(7000 + seed, c["batch"], c["dim"], c["L"], dstate=c["dstate"], device=DEV,
                                  gated=c["gated"], perturb=True, bc_layout=c["bc_layout"])
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(7100 + seed, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=0.5, zoh=c["zoh"])
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(host_dir(fwd), host_dir(bwd), host(dout), z=host(z),
                                           combine_scale=0.5, zoh=c["zoh"])
    for k in _GRAD_KEYS:
        if k == "delta_bias" and wf[k] is None:
            continue
        assert_close(host(gf[k]), wf[k], FP32_TOL, f"fwd d{k}")
        assert_close(host(gb[k]), wb[k], FP32_TOL, f"bwd d{k}")
    if z is not None:
        assert_close(host(dz), wdz, FP32_TOL, "dz")


def _draw_map(seed, max_side):
    r = random.Random(seed)
    H, W = r.randint(1, max_side), r.randint(1, max_side)
    if r.random() < 0.5:                     # the four-wide layout kernels
        H, W = 4 * ((H + 3) // 4), 4 * ((W + 3) // 4)
    return dict(H=H, W=W, batch=r.choice([1, 2, 3]), dim=r.choice([1, 5, 16, 23, 40]),
                dstate=r.choice([16, 16, 11, 4]), zoh=r.random() < 0.3, bf16=r.random() < 0.25,
                gated=r.random() < 0.8, bc_layout=r.choice(["token", "dense"]), axis=r.choice([0, 1]),
                bidir=r.random() < 0.7)


@pytest.mark.parametrize("seed", range(8))
def test_random_es2d(seed):
    c = _draw_map(4000 + seed, 40)
    _case(f"random es2d {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    batch, dim, H, W = c["batch"], c["dim"], c["H"], c["W"]
    x, p = wl.es2d_inputs(8000 + seed, batch, dim, H, W, dstate=c["dstate"], device=DEV, dtype=dt,
                          perturb=True, bc_layout=c["bc_layout"])
    s = vm.vm_atrous_gather(x)
    Lg = s.shape[-1]
    y = vm.vm_selective_scan_fwd(s.reshape(4 * batch, dim, Lg), **p, zoh=c["zoh"])
    out = vm.vm_atrous_scatter(y.reshape(batch, 4, dim, Lg), H, W)
    torch.cuda.synchronize()
    hs = oracle.atrous_gather(host(x))
    assert np.array_equal(host(s), hs), "gather is a bit-exact copy"
    assert np.array_equal(host(out), oracle.atrous_scatter(host(y).reshape(batch, 4, dim, Lg), H, W)), \
        "scatter is a bit-exact copy"
    hy = oracle.selective_scan(hs.reshape(4 * batch, dim, Lg), **host_dir(p), zoh=c["zoh"])
    ref = oracle.atrous_scatter(hy.reshape(batch, 4, dim, Lg), H, W)
    assert_close(host(out), ref, BF16_TOL if c["bf16"] else FP32_TOL, "random es2d")


@pytest.mark.parametrize("seed", range(8))
def test_random_ss2d(seed):
    c = _draw_map(4100 + seed, 40)
    _case(f"random ss2d {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    u, dirs, z = wl.ss2d_inputs(8100 + seed, c["batch"], c["dim"], c["H"], c["W"], dstate=c["dstate"],
                                device=DEV, dtype=dt, gated=c["gated"], perturb=True, bc_layout=c["bc_layout"])
    out = vm.vm_ss2d_scan_fwd(u, dirs, z=z, combine_scale=0.5, zoh=c["zoh"])
    torch.cuda.synchronize()
    ref = oracle.ss2d_scan(host(u), [host_dir(p) for p in dirs], z=host(z), combine_scale=0.5, zoh=c["zoh"])
    assert_close(host(out), ref, BF16_TOL if c["bf16"] else FP32_TOL, "random ss2d")


@pytest.mark.parametrize("seed", range(6))
def test_random_ss2d_bwd(seed):
    # maps of at most 16 x 16 (the gradient oracle walks every step in Python)
    c = _draw_map(4200 + seed, 16)
    _case(f"random ss2d bwd {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    u, dirs, z = wl.ss2d_inputs(8200 + seed, c["batch"], c["dim"], c["H"], c["W"], dstate=c["dstate"],
                                device=DEV, dtype=dt, gated=c["gated"], perturb=True, bc_layout=c["bc_layout"])
    dout = torch.randn(u.shape, generator=wl.generator(8300 + seed, DEV), device=DEV).to(dt)
    du, grads, dz = vm.vm_ss2d_scan_bwd(u, dirs, dout, z=z, combine_scale=0.5, zoh=c["zoh"])
    torch.cuda.synchronize()
    wdu, wg, wdz, _ = ograd.ss2d_scan_grad(host(u), [host_dir(p) for p in dirs], host(dout), z=host(z),
                                           combine_scale=0.5, zoh=c["zoh"])
    # the pass runs in fp32 on the exact widening of bf16 inputs
    assert_close(host(du), wdu, FP32_TOL, "du")
    for k in range(4):
        for key in _GRAD_KEYS[1:]:
            if wg[k][key] is None:
                assert grads[k][key] is None
            else:
                assert_close(host(grads[k][key]), wg[k][key], FP32_TOL, f"dir{k} d{key}")
    if z is None:
        assert dz is None
    else:
        assert_close(host(dz), wdz, FP32_TOL, "dz")


@pytest.mark.parametrize("seed", range(8))
def test_random_pool_scan_repeat(seed):
    c = _draw_map(4300 + seed, 40)
    _case(f"random pooled {c}")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    fwd, bwd, z = wl.fastvim_inputs(8400 + seed, c["batch"], c["dim"], c["H"], c["W"], c["axis"],
                                    dstate=c["dstate"], device=DEV, dtype=dt, perturb=True,
                                    bc_layout=c["bc_layout"])
    z = z if c["gated"] else None
    b = bwd if c["bidir"] else None
    out = vm.vm_pool_scan_repeat(fwd, b, z=z, combine_scale=0.5, pool_axis=c["axis"], zoh=c["zoh"])
    torch.cuda.synchronize()
    ref = oracle.pool_scan_repeat(host_dir(fwd), host_dir(b) if b is not None else None, z=host(z),
                                  combine_scale=0.5, pool_axis=c["axis"], zoh=c["zoh"])
    assert_close(host(out), ref, BF16_TOL if c["bf16"] else FP32_TOL, "random pooled")


@pytest.mark.parametrize("seed", range(6))
def test_random_pool_scan_repeat_bwd(seed):
    c = _draw_map(4400 + seed, 40)
    c["bf16"] = False
    _case(f"random pooled bwd {c}")
    fwd, bwd, z = wl.fastvim_inputs(8500 + seed, c["batch"], c["dim"], c["H"], c["W"], c["axis"],
                                    dstate=c["dstate"], device=DEV, perturb=True, bc_layout=c["bc_layout"])
    z = z if c["gated"] else None
    b = bwd if c["bidir"] else None
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(8600 + seed, DEV), device=DEV)
    gf, gb, dz = vm.vm_pool_scan_repeat_bwd(fwd, dout, bwd=b, z=z, combine_scale=0.5, pool_axis=c["axis"],
                                            zoh=c["zoh"])
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.pool_scan_repeat_grad(host_dir(fwd), host_dir(b) if b is not None else None,
                                                 host(dout), z=host(z), combine_scale=0.5,
                                                 pool_axis=c["axis"], zoh=c["zoh"])
    for got, want, tag in ((gf, wf, "fwd"), (gb, wb, "bwd")):
        if want is None:
            assert got is None
            continue
        for k in _GRAD_KEYS:
            if k == "delta_bias" and want[k] is None:
                continue
            assert_close(host(got[k]), want[k], FP32_TOL, f"{tag} d{k}")
    if z is None:
        assert dz is None
    else:
        assert_close(host(dz), wdz, FP32_TOL, "dz")
