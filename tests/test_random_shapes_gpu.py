"""Seeded random shapes and options through the C ABI against the oracles:
forward single and bidirectional scans, and the bidirectional backward.  The
draws cover the planner's branches (sequence-parallel single scan, 4- and
8-lane splits, on-chip and global exchange, workgroups of one or two row
blocks), ragged tiles, partial row blocks, dstate below 16, both B/C layouts,
the zero-order-hold write, the fused conv, bf16 and the ungated scan."""
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
