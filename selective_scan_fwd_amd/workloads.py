"""Seeded synthetic workloads for the selective-scan hot path.

This module only draws random tensors of the pages' shapes and value
distributions; it performs none of the method's arithmetic.  Both the HIP
path (tests, benchmark) and the oracle (tests, CPU baseline) take their
inputs from here.  Draws use torch's generator on the requested device, so a
seed reproduces the same tensors on the same device type.

Distributions (the same for every workload):
  u, delta, z, B, C ~ N(0, 1)           (fp32 draws; bf16 workloads round
                                          them to nearest even)
  delta_bias[d]    = -4.6 + U(-0.5, 0.5) per channel and direction, so that
                     dt = softplus(delta + bias) falls mostly in [1e-3, 1e-1]
  A[d, n]          = -(n + 1)            (S4D-real decay; A = -exp(A_log))
  D[d]             = 1
``perturb=True`` multiplies A by (1 + 0.25 U(0,1)) and D by (1 + 0.25 N(0,1))
per element so that parity tests catch swapped directions or parameters.

B and C are returned with shape [batch, N, L] as the pages index them.  With
``bc_layout="token"`` (the default) they are transposed views of token-major
[batch, L, N] storage, which is how the page's projection produces them (it
splits the projected tokens and passes transposed views to the scan); with
``bc_layout="dense"`` they are contiguous [batch, N, L] tensors.

Token geometry (Vision Mamba page, "From pixels to position-aware tokens"):
a 224x224 image with 16x16 windows gives 14x14 = 196 patches plus a middle
CLS token, L = 197; a 1024x1024 image gives 64x64 + 1 = 4097.
"""
from __future__ import annotations

import dataclasses

import torch

DSTATE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "single" | "bidir" | "es2d" | "fastvim" | "ss2d"
    dtype: str           # "f32" | "bf16"
    batch: int
    dim: int
    seqlen: int = 0      # single / bidir
    sizes: tuple = ()    # es2d: square map sizes
    height: int = 0      # fastvim / ss2d grid
    width: int = 0
    gated: bool = True
    combine_scale: float = 1.0


def patch_tokens(image: int, patch: int, stride: int) -> int:
    """Patch count per side squared, plus one CLS token."""
    side = (image - patch) // stride + 1
    return side * side + 1


WORKLOADS = {
    0: Workload(0, "single_fp32_b1_l197_d384", "single", "f32", 1, 384, seqlen=patch_tokens(224, 16, 16)),
    1: Workload(1, "vim_t_bidir_fp32_b128_l197_d384", "bidir", "f32", 128, 384,
                seqlen=patch_tokens(224, 16, 16)),
    2: Workload(2, "vim_s_bidir_bf16_b16_l4097_d768", "bidir", "bf16", 16, 768,
                seqlen=patch_tokens(1024, 16, 16)),
    3: Workload(3, "es2d_fp32_b64_c192_56_57", "es2d", "f32", 64, 192, sizes=(56, 57), gated=False),
    4: Workload(4, "fastvim_fp32_b128_d384_128x128", "fastvim", "f32", 128, 384, height=128, width=128),
    # dense four-direction counterpart of the ES2D stage above (same map and channels)
    5: Workload(5, "ss2d_fp32_b64_c192_56x56", "ss2d", "f32", 64, 192, height=56, width=56),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, device, dtype):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def _bc_pair(g, batch, dstate, L, device, dtype, bc_layout):
    """B, C of shape [batch, dstate, L] in the requested storage layout."""
    if bc_layout == "token":
        B = _normal(g, (batch, L, dstate), device, dtype).transpose(1, 2)
        C = _normal(g, (batch, L, dstate), device, dtype).transpose(1, 2)
    elif bc_layout == "dense":
        B = _normal(g, (batch, dstate, L), device, dtype)
        C = _normal(g, (batch, dstate, L), device, dtype)
    else:
        raise ValueError(bc_layout)
    return B, C


def scan_params(g, dim, dstate=DSTATE, device="cpu", perturb=False):
    """A [dim, dstate], D [dim], delta_bias [dim] (always fp32)."""
    A = -torch.arange(1, dstate + 1, device=device, dtype=torch.float32).repeat(dim, 1)
    D = torch.ones(dim, device=device, dtype=torch.float32)
    bias = -4.6 + (torch.rand(dim, generator=g, device=device, dtype=torch.float32) - 0.5)
    if perturb:
        A = A * (1.0 + 0.25 * torch.rand(A.shape, generator=g, device=device))
        D = D * (1.0 + 0.25 * torch.randn(D.shape, generator=g, device=device))
    return A.contiguous(), D.contiguous(), bias.contiguous()


def conv_params(g, dim, device="cpu"):
    """Depthwise width-4 conv weights [dim, 4] and bias [dim] (fp32), drawn
    U(-0.5, 0.5) like a fan-in-4 uniform initialisation."""
    w = torch.rand((dim, 4), generator=g, device=device, dtype=torch.float32) - 0.5
    b = torch.rand((dim,), generator=g, device=device, dtype=torch.float32) - 0.5
    return w.contiguous(), b.contiguous()


def scan_direction(g, batch, dim, seqlen, dstate=DSTATE, device="cpu", dtype=torch.float32,
                   perturb=False, u_shape=None, delta_len=None, bc_layout="token"):
    """One direction's tensors: u, delta [batch, dim, L]; B, C [batch, dstate, L];
    A, D, delta_bias.  u_shape / delta_len override the u shape and the length
    of delta/B/C (FastVim: full-resolution u, pooled delta/B/C)."""
    L = seqlen if delta_len is None else delta_len
    u = _normal(g, u_shape or (batch, dim, seqlen), device, dtype)
    delta = _normal(g, (batch, dim, L), device, dtype)
    B, C = _bc_pair(g, batch, dstate, L, device, dtype, bc_layout)
    A, D, bias = scan_params(g, dim, dstate, device, perturb)
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=bias)


def single_inputs(seed, batch, dim, seqlen, dstate=DSTATE, device="cpu", dtype=torch.float32,
                  gated=True, perturb=False, bc_layout="token"):
    g = generator(seed, device)
    p = scan_direction(g, batch, dim, seqlen, dstate, device, dtype, perturb, bc_layout=bc_layout)
    z = _normal(g, (batch, dim, seqlen), device, dtype) if gated else None
    return p, z


def bidir_inputs(seed, batch, dim, seqlen, dstate=DSTATE, device="cpu", dtype=torch.float32,
                 gated=True, perturb=False, bc_layout="token"):
    """Forward then backward direction (each with its own parameters), then z."""
    g = generator(seed, device)
    fwd = scan_direction(g, batch, dim, seqlen, dstate, device, dtype, False, bc_layout=bc_layout)
    bwd = scan_direction(g, batch, dim, seqlen, dstate, device, dtype, perturb, bc_layout=bc_layout)
    z = _normal(g, (batch, dim, seqlen), device, dtype) if gated else None
    return fwd, bwd, z


def es2d_inputs(seed, batch, channels, height, width, dstate=DSTATE, device="cpu",
                dtype=torch.float32, perturb=False, bc_layout="token"):
    """Feature map x [batch, channels, H, W] and the per-group scan's delta
    [4*batch, channels, Lg] and B, C [4*batch, dstate, Lg], drawn directly in
    gathered layout (pad steps included), plus A, D, delta_bias."""
    g = generator(seed, device)
    Lg = ((height + 1) // 2) * ((width + 1) // 2)
    x = _normal(g, (batch, channels, height, width), device, dtype)
    delta = _normal(g, (4 * batch, channels, Lg), device, dtype)
    B, C = _bc_pair(g, 4 * batch, dstate, Lg, device, dtype, bc_layout)
    A, D, bias = scan_params(g, channels, dstate, device, perturb)
    return x, dict(delta=delta, A=A, B=B, C=C, D=D, delta_bias=bias)


def fastvim_inputs(seed, batch, dim, height, width, pool_axis, dstate=DSTATE, device="cpu",
                   dtype=torch.float32, perturb=False, full_resolution=False, bc_layout="token"):
    """Per direction: full-resolution u [batch, dim, H, W], and delta, B, C
    drawn at full resolution ([batch, dim, H*W] and [batch, dstate, H*W],
    rows slow and columns fast); then z [batch, dim, H, W].  The pooled scan
    (full_resolution=False) takes their means along the pooled axis (over W
    for pool_axis 0, giving length H; over H for axis 1): a linear projection
    commutes with the mean, so these are the projections of the pooled
    tokens, and the pooled and unpooled paths run on the same seeded
    tensors.  full_resolution=True returns delta, B, C unpooled."""
    g = generator(seed, device)
    L = height * width

    def pooled(t, rows):                      # [batch, rows, H*W] -> [batch, rows, Lp], fp32 mean
        m = t.float().reshape(batch, rows, height, width).mean(dim=3 if pool_axis == 0 else 2)
        return m.to(dtype)

    def pooled_bc(t):
        m = pooled(t, dstate)                 # [batch, dstate, Lp]
        if bc_layout == "token":              # token-major storage, viewed as [batch, dstate, Lp]
            return m.transpose(1, 2).contiguous().transpose(1, 2)
        return m.contiguous()

    dirs = []
    for k in range(2):
        u = _normal(g, (batch, dim, height, width), device, dtype)
        delta = _normal(g, (batch, dim, L), device, dtype)
        B, C = _bc_pair(g, batch, dstate, L, device, dtype, bc_layout)
        A, D, bias = scan_params(g, dim, dstate, device, perturb and k == 1)
        if not full_resolution:
            delta = pooled(delta, dim).contiguous()
            B, C = pooled_bc(B), pooled_bc(C)
        dirs.append(dict(u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=bias))
    z = _normal(g, (batch, dim, height, width), device, dtype)
    return dirs[0], dirs[1], z


def ss2d_inputs(seed, batch, dim, height, width, dstate=DSTATE, device="cpu", dtype=torch.float32,
                gated=True, perturb=False, bc_layout="token"):
    """Feature map u [batch, dim, H, W], four traversals' delta [batch, dim,
    H*W], B, C [batch, dstate, H*W] (drawn in each traversal's own step
    order), A, D, delta_bias, then z [batch, dim, H, W].  perturb applies to
    traversals 1 and 3, so that the four parameter sets differ."""
    g = generator(seed, device)
    L = height * width
    u = _normal(g, (batch, dim, height, width), device, dtype)
    dirs = []
    for k in range(4):
        delta = _normal(g, (batch, dim, L), device, dtype)
        B, C = _bc_pair(g, batch, dstate, L, device, dtype, bc_layout)
        A, D, bias = scan_params(g, dim, dstate, device, perturb and k % 2 == 1)
        dirs.append(dict(delta=delta, A=A, B=B, C=C, D=D, delta_bias=bias))
    z = _normal(g, (batch, dim, height, width), device, dtype) if gated else None
    return u, dirs, z
