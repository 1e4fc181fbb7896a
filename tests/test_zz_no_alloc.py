"""The no-allocation entry point vm_bidir_scan_fwd_noalloc, through the C
ABI: its output equals vm_bidir_scan_fwd's (the same kernels) bit for bit,
on two calls in a row, the second smaller, where the exchange buffer is the
library-owned device array (bf16, and fp32 with a sequence length that is
not a multiple of 32), and where out serves as the exchange."""
import sys

import pytest
import torch

import selective_scan_fwd_amd as vm
from selective_scan_fwd_amd import workloads as wl

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


def _pair(seed, batch, dim, L, dtype, zoh=False):
    fwd, bwd, z = wl.bidir_inputs(seed, batch, dim, L, device=DEV, dtype=dtype, perturb=True)
    ref = vm.vm_bidir_scan_fwd(fwd, bwd, z=z, combine_scale=0.5, zoh=zoh)
    out = torch.full_like(ref, float("nan"))
    got = vm.vm_bidir_scan_fwd_noalloc(fwd, bwd, out, z=z, combine_scale=0.5, zoh=zoh)
    torch.cuda.synchronize()
    assert got is out
    return got, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_bidir_twice_second_smaller(dtype):
    # 600 and 577 steps: past the on-chip exchange (552), and not multiples of
    # 32, so the exchange rows live in the library-owned array
    for seed, batch, dim, L in ((11, 3, 70, 600), (12, 2, 33, 577)):
        _case(f"noalloc bidir {dtype} b{batch} d{dim} L{L}")
        got, ref = _pair(seed, batch, dim, L, dtype)
        assert torch.equal(got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_noalloc_short_and_out_as_exchange():
    # on-chip exchange (197 steps), and fp32 with 608 steps (out is the exchange)
    for seed, L, zoh in ((21, 197, False), (22, 608, True)):
        _case(f"noalloc bidir fp32 L{L} zoh{zoh}")
        got, ref = _pair(seed, 2, 40, L, torch.float32, zoh=zoh)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_noalloc_rejects_past_its_array():
    # 4 x 512 rows x 4128 (4097 rounded up) fp32 values exceed 8 Mi: rejected
    _case("noalloc rejects an exchange past the array")
    fwd, bwd, z = wl.bidir_inputs(31, 4, 512, 4097, device=DEV, dtype=torch.bfloat16)
    out = torch.empty_like(z)
    with pytest.raises(vm.VmError):
        vm.vm_bidir_scan_fwd_noalloc(fwd, bwd, out, z=z)
