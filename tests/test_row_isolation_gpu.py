"""Rows of a scan are independent: a channel's output depends on its own
(u, Δ) row only.  The scan kernels load a ragged last tile with plain
offsets, so the steps past L of one row read the first values of the next
row; those values may only reach states after the row's last real step.
Here every odd channel starts with non-finite or huge values, and every even
channel must still match the oracle exactly (to the fp32 bound), for the
one-direction scan both ways, the bidirectional scan with the on-chip and
with the global exchange, and the backward of the bidirectional scan."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_fwd_amd as vm
from oracle import grad as ograd
from selective_scan_fwd_amd import workloads as wl

from _helpers import FP32_TOL, assert_close, host, host_dir

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _poison(p, head):
    """Odd channels: the first `head` steps of u and Δ become inf, nan and
    1e30 in turn (even channels untouched)."""
    for k, bad in (("u", float("inf")), ("delta", float("nan"))):
        v = p[k]
        v[:, 1::2, :head] = bad
        v[:, 1::4, :head] = 1e30


def _even(a):
    return a[:, 0::2]


def _even_dir(h):
    out = dict(h)
    out["u"], out["delta"] = _even(h["u"]), _even(h["delta"])
    for k in ("A", "D", "delta_bias"):
        if out.get(k) is not None:
            out[k] = h[k][0::2]
    return out


@pytest.mark.parametrize("L,reverse", [(197, False), (197, True), (23, False), (600, True), (601, False)])
def test_single_rows_isolated(L, reverse):
    print(f"[case] single L={L} reverse={reverse}", flush=True)
    p, z = wl.single_inputs(7100 + L, 2, 34, L, device=DEV)
    _poison(p, 16)
    out = vm.vm_selective_scan_fwd(**p, z=z, reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(**_even_dir(host_dir(p)), z=_even(host(z)), reverse=reverse)
    assert_close(_even(host(out)), ref, FP32_TOL, "single, even rows")


@pytest.mark.parametrize("L", [197, 31, 553, 650])
def test_bidir_rows_isolated(L):
    print(f"[case] bidir L={L}", flush=True)
    fwd, bwd, z = wl.bidir_inputs(7200 + L, 2, 34, L, device=DEV)
    _poison(fwd, 16)
    _poison(bwd, 16)
    out = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5)
    torch.cuda.synchronize()
    ref = oracle.bidir_scan(_even_dir(host_dir(fwd)), _even_dir(host_dir(bwd)), z=_even(host(z)),
                            combine_scale=0.5)
    assert_close(_even(host(out)), ref, FP32_TOL, "bidir, even rows")


@pytest.mark.parametrize("L", [197, 650])
def test_bidir_bwd_rows_isolated(L):
    print(f"[case] bidir backward L={L}", flush=True)
    fwd, bwd, z = wl.bidir_inputs(7300 + L, 1, 34, L, device=DEV)
    _poison(fwd, 16)
    _poison(bwd, 16)
    dout = torch.randn(fwd["u"].shape, generator=wl.generator(7350 + L, DEV), device=DEV)
    gf, gb, dz = vm.vm_bidir_scan_bwd(fwd, bwd, dout, z=z, combine_scale=1.0)
    torch.cuda.synchronize()
    wf, wb, wdz, _ = ograd.bidir_scan_grad(_even_dir(host_dir(fwd)), _even_dir(host_dir(bwd)),
                                           _even(host(dout)), z=_even(host(z)), combine_scale=1.0)
    # dB and dC sum over all channels (the poisoned ones too); the rest is per channel
    for got, want, tag in ((gf, wf, "fwd"), (gb, wb, "bwd")):
        for k in ("u", "delta"):
            assert_close(_even(host(got[k])), want[k], FP32_TOL, f"{tag} d{k}, even rows")
        for k in ("A", "D", "delta_bias"):
            assert_close(host(got[k])[0::2], want[k], FP32_TOL, f"{tag} d{k}, even channels")
    assert_close(_even(host(dz)), wdz, FP32_TOL, "dz, even rows")
