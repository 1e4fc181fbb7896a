"""CPU checks of the seeded workload generator: shapes from the pages' token
geometry, determinism, and the step-size distribution the recipe promises."""
import json
import os

import torch

from selective_scan_fwd_amd import workloads as wl


def test_token_geometry_matches_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "token_geometry.json")))
    for c in g["cases"]:
        assert wl.patch_tokens(c["image"], c["patch"], c["stride"]) == c["tokens"]
        assert c["cls_index"] == c["patches"] // 2
    assert wl.WORKLOADS[1].seqlen == 197
    assert wl.WORKLOADS[2].seqlen == 64 * 64 + 1


def test_seeded_and_deterministic():
    a = wl.bidir_inputs(5, 2, 8, 11)
    b = wl.bidir_inputs(5, 2, 8, 11)
    for x, y in zip(list(a[0].values()) + list(a[1].values()) + [a[2]],
                    list(b[0].values()) + list(b[1].values()) + [b[2]]):
        assert torch.equal(x, y)
    c = wl.bidir_inputs(6, 2, 8, 11)
    assert not torch.equal(a[0]["u"], c[0]["u"])


def test_step_size_mostly_in_range():
    fwd, bwd, _ = wl.bidir_inputs(1001, 8, 384, 197)
    for p in (fwd, bwd):
        dt = torch.nn.functional.softplus(p["delta"] + p["delta_bias"][None, :, None])
        frac = ((dt >= 1e-3) & (dt <= 1e-1)).float().mean().item()
        assert frac >= 0.9, frac
    assert torch.equal(fwd["A"][0], -torch.arange(1, 17, dtype=torch.float32))


def test_bf16_rounding_and_shapes():
    fwd, bwd, z = wl.bidir_inputs(3, 2, 4, 9, dtype=torch.bfloat16)
    assert fwd["u"].dtype == torch.bfloat16 and fwd["A"].dtype == torch.float32
    x, p = wl.es2d_inputs(2, 2, 3, 5, 7)
    assert x.shape == (2, 3, 5, 7) and p["delta"].shape == (8, 3, 12) and p["B"].shape == (8, 16, 12)
    f, b, z = wl.fastvim_inputs(4, 2, 3, 4, 6, pool_axis=1)
    assert f["u"].shape == (2, 3, 4, 6) and f["delta"].shape == (2, 3, 6) and f["B"].shape == (2, 16, 6)
    F, Bk, Z = wl.fastvim_inputs(4, 2, 3, 4, 6, pool_axis=1, full_resolution=True)
    assert F["delta"].shape == (2, 3, 24) and F["B"].shape == (2, 16, 24)
    # the pooled inputs are the means of the same seeded full-resolution
    # draws (over H for axis 1), and u, z and the parameters are shared
    assert torch.equal(f["u"], F["u"]) and torch.equal(z, Z) and torch.equal(f["A"], F["A"])
    torch.testing.assert_close(f["delta"], F["delta"].reshape(2, 3, 4, 6).mean(2), rtol=0, atol=1e-6)
    torch.testing.assert_close(f["B"], F["B"].reshape(2, 16, 4, 6).mean(2), rtol=0, atol=1e-6)
    torch.testing.assert_close(b["C"], Bk["C"].reshape(2, 16, 4, 6).mean(2), rtol=0, atol=1e-6)
    assert f["B"].stride(1) == 1                       # token-major storage, as the unpooled B
    f0, _, _ = wl.fastvim_inputs(4, 2, 3, 4, 6, pool_axis=0)
    torch.testing.assert_close(f0["delta"], F["delta"].reshape(2, 3, 4, 6).mean(3), rtol=0, atol=1e-6)


def test_ss2d_and_conv_generators():
    u, dirs, z = wl.ss2d_inputs(7, 2, 3, 5, 4)
    assert u.shape == (2, 3, 5, 4) and z.shape == u.shape and len(dirs) == 4
    for p in dirs:
        assert "u" not in p and p["delta"].shape == (2, 3, 20) and p["B"].shape == (2, 16, 20)
    # four distinct draws of the per-traversal inputs
    assert not torch.equal(dirs[0]["delta"], dirs[2]["delta"])
    w = wl.WORKLOADS[5]
    assert (w.height, w.width, w.batch, w.dim) == (56, 56, 64, 192)
    g = wl.generator(3, "cpu")
    cw, cb = wl.conv_params(g, 10)
    assert cw.shape == (10, 4) and cb.shape == (10,)
    assert cw.abs().max().item() <= 0.5 and cb.abs().max().item() <= 0.5
