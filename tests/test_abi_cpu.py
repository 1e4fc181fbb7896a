"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and its host-side argument checks return the documented
status codes without launching anything (no GPU is touched on these paths)."""
import ctypes
import os
import re

import pytest

import selective_scan_fwd_amd as vm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vm_scan.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vm_[a-z0-9_]+)\s*\(", src)))


def _status_codes():
    src = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(VM_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vm.LIB_PATH):
        from selective_scan_fwd_amd import build
        build.build()
    return vm.load_library()


def test_exports_match_header(lib):
    declared = _declared_functions()
    assert set(declared) == set(vm.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    codes = _status_codes()
    assert codes["VM_OK"] == 0 and len(codes) == len(vm.STATUS_NAMES)
    for name, code in codes.items():
        assert vm.STATUS_NAMES[code] == name
        assert vm.vm_status_string(code).startswith(name)
    assert vm.vm_status_string(999) == "unknown status"
    assert vm.vm_version() >= 10000


def test_group_len(lib):
    assert vm.vm_atrous_group_len(56, 56) == 784
    assert vm.vm_atrous_group_len(57, 57) == 841
    assert vm.vm_atrous_group_len(3, 5) == 6
    assert vm.vm_atrous_group_len(1, 1) == 1
    assert lib.vm_atrous_group_len(0, 4) == -2
    assert lib.vm_atrous_group_len(4, -1) == -2


FAKE = 1 << 40          # plausible-looking but never dereferenced device addresses


def _dir(base):
    # non-overlapping fake pointers: each tensor gets its own 2^32-byte window
    return vm.VmScanDir(*(base + k * (1 << 32) for k in range(7)))


def _scan(lib, d=None, z=None, out=FAKE * 3, batch=2, dim=4, L=5, N=16, dtype=0, sp=1, rev=0):
    d = _dir(FAKE) if d is None else d
    return lib.vm_selective_scan_fwd(ctypes.byref(d), z, out, batch, dim, L, N, dtype, sp, rev, None)


def test_scan_argument_checks(lib):
    assert lib.vm_selective_scan_fwd(None, None, FAKE * 3, 2, 4, 5, 16, 0, 1, 0, None) == 1
    assert _scan(lib, out=None) == 1
    d = _dir(FAKE)
    d.B = None
    assert _scan(lib, d=d) == 1
    d = _dir(FAKE)
    d.D = None
    assert _scan(lib, d=d) == 1
    assert _scan(lib, batch=0) == 2
    assert _scan(lib, dim=-3) == 2
    assert _scan(lib, L=0) == 2
    assert _scan(lib, N=0) == 2
    assert _scan(lib, batch=1 << 40, dim=1 << 20) == 2          # element count overflow
    assert _scan(lib, N=17) == 6
    assert _scan(lib, batch=1, L=1 << 26) == 6                  # past the 32-bit in-kernel offsets
    assert _scan(lib, dtype=2) == 3
    assert _scan(lib, sp=4) == 4                                # unknown option bit
    assert _scan(lib, sp=-1) == 4
    assert _scan(lib, rev=-1) == 4
    # output overlapping an input
    d = _dir(FAKE)
    assert _scan(lib, d=d, out=d.u) == 5
    assert _scan(lib, d=d, out=d.delta + 8) == 5
    assert _scan(lib, d=d, out=d.B) == 5
    assert _scan(lib, z=FAKE * 3, out=FAKE * 3) == 5
    # token-major B / C: stride must cover dstate; overlap uses the strided extent
    d = _dir(FAKE)
    d.bc_stride = -1
    assert _scan(lib, d=d) == 2
    d.bc_stride = 15
    assert _scan(lib, d=d) == 2
    d = _dir(FAKE)
    d.bc_stride = 1 << 20                 # B extent = (2*5-1) * 2^20 + 16 elements
    assert _scan(lib, d=d, out=d.B + 4 * (9 << 20)) == 5


def test_bidir_argument_checks(lib):
    f, b = _dir(FAKE), _dir(FAKE * 2)

    def call(fwd=f, bwd=b, z=None, scale=1.0, out=FAKE * 3, N=16, dtype=0, sp=1):
        pf = ctypes.byref(fwd) if fwd is not None else None
        pb = ctypes.byref(bwd) if bwd is not None else None
        return lib.vm_bidir_scan_fwd(pf, pb, z, scale, out, 2, 4, 5, N, dtype, sp, None)

    assert call(fwd=None) == 1
    assert call(bwd=None) == 1
    assert call(scale=float("nan")) == 6
    assert call(scale=float("inf")) == 6
    assert call(N=32) == 6
    assert call(dtype=-1) == 3
    assert call(sp=8) == 4
    assert call(out=b.C) == 5


def test_bidir_noalloc_argument_checks(lib):
    # the same checks as vm_bidir_scan_fwd, then the bound of its exchange
    # array: 4 x 512 rows x 4128 (4097 rounded up to 32) fp32 values > 8 Mi,
    # rejected on the host before any HIP call
    f, b = _dir(FAKE), _dir(FAKE * 2)

    def call(out=FAKE * 3, batch=2, dim=4, L=5, N=16, dtype=0, scale=1.0):
        return lib.vm_bidir_scan_fwd_noalloc(ctypes.byref(f), ctypes.byref(b), None, scale, out, batch, dim, L,
                                             N, dtype, 1, None)

    assert call(out=None) == 1
    assert call(dtype=3) == 3
    assert call(N=0) == 2
    assert call(N=17) == 6
    assert call(scale=float("nan")) == 6
    assert call(out=f.u) == 5
    assert call(batch=4, dim=512, L=4097, dtype=1) == 6


def test_atrous_argument_checks(lib):
    assert lib.vm_atrous_gather(None, FAKE * 3, 1, 1, 4, 4, 0, None) == 1
    assert lib.vm_atrous_gather(FAKE, None, 1, 1, 4, 4, 0, None) == 1
    assert lib.vm_atrous_gather(FAKE, FAKE * 3, 1, 1, 0, 4, 0, None) == 2
    assert lib.vm_atrous_gather(FAKE, FAKE * 3, 1, 1, 4, 4, 5, None) == 3
    assert lib.vm_atrous_gather(FAKE, FAKE + 16, 1, 1, 4, 4, 0, None) == 5
    assert lib.vm_atrous_scatter(FAKE, FAKE * 3, 1, 0, 4, 4, 0, None) == 2
    assert lib.vm_atrous_scatter(FAKE, None, 1, 1, 4, 4, 0, None) == 1
    assert lib.vm_atrous_scatter(FAKE, FAKE + 60, 1, 1, 4, 4, 0, None) == 5


def test_pool_argument_checks(lib):
    f, b = _dir(FAKE), _dir(FAKE * 2)

    def call(fwd=f, bwd=b, axis=0, H=8, W=6, N=16, out=FAKE * 3, sp=1, dtype=0, scale=0.5):
        pf = ctypes.byref(fwd) if fwd is not None else None
        pb = ctypes.byref(bwd) if bwd is not None else None
        return lib.vm_pool_scan_repeat(pf, pb, None, scale, out, 2, 4, H, W, N, axis, dtype, sp, None)

    assert call(fwd=None) == 1
    assert call(axis=2) == 4
    assert call(H=0) == 2
    assert call(N=0) == 2
    assert call(N=20) == 6
    assert call(scale=float("nan")) == 6
    assert call(dtype=9) == 3
    assert call(out=f.u + 4) == 5


def test_ss2d_argument_checks(lib):
    dirs = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))

    def call(d=dirs, u=FAKE, z=None, scale=1.0, out=FAKE * 3, H=6, W=5, N=16, dtype=0, sp=1):
        return lib.vm_ss2d_scan_fwd(d, u, z, scale, out, 2, 4, H, W, N, dtype, sp, None)

    assert call(d=None) == 1
    assert call(u=None) == 1
    assert call(out=None) == 1
    bad = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))
    bad[3].C = None
    assert call(d=bad) == 1
    bad = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))
    bad[2].u = None                          # ignored (every traversal reads u): the call
    assert call(d=bad, z=FAKE * 3) == 5      # gets past the pointer checks to the z alias
    assert call(H=0) == 2
    assert call(W=-1) == 2
    assert call(N=0) == 2
    assert call(N=17) == 6
    assert call(scale=float("nan")) == 6
    assert call(H=40000, W=40000) == 6       # more than 65535 tiles of 32 x 32 pixels
    assert call(dtype=4) == 3
    assert call(sp=-1) == 4
    assert call(out=FAKE + 8) == 5           # overlaps u
    assert call(out=dirs[2].delta) == 5
    assert call(out=dirs[1].B + 4) == 5
    assert call(z=FAKE * 3, out=FAKE * 3) == 5


def test_plane_count_limit(lib):
    # map kernels run one workgroup per plane on grid x: at most 2^24 - 1 planes
    big = 1 << 12
    assert lib.vm_atrous_gather(FAKE, FAKE * 3, big, big, 2, 2, 0, None) == 6
    assert lib.vm_atrous_scatter(FAKE, FAKE * 3, big, big, 2, 2, 0, None) == 6
    f = _dir(FAKE)
    assert lib.vm_pool_scan_repeat(ctypes.byref(f), None, None, 1.0, FAKE * 3, big, big, 2, 2, 16,
                                   0, 0, 1, None) == 6
    dirs = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))
    assert lib.vm_ss2d_scan_fwd(dirs, FAKE, None, 1.0, FAKE * 3, big, big, 2, 2, 16, 0, 1, None) == 6


def test_pool_bwd_argument_checks(lib):
    f, b = _dir(FAKE), _dir(FAKE * 2)
    gf = vm.VmScanGrad(*(FAKE * 5 + k * (1 << 32) for k in range(9)))
    gb = vm.VmScanGrad(*(FAKE * 6 + k * (1 << 32) for k in range(9)))

    def call(fb=None, z=None, dout=FAKE * 3, g2=None, dz=None, axis=0, dtype=0, scale=1.0, N=16):
        return lib.vm_pool_scan_repeat_bwd(ctypes.byref(f), fb, z, dout, scale, ctypes.byref(gf), g2, dz,
                                           2, 4, 6, 8, N, axis, dtype, 1, None)

    assert call(dout=None) == 1
    assert call(z=FAKE * 4) == 1                            # z without dz
    assert call(fb=ctypes.byref(b)) == 1                    # bwd without its gradients
    assert call(axis=2) == 4
    assert call(dtype=4) == 3
    assert call(N=17) == 6
    assert call(scale=float("nan")) == 6
    assert call(z=FAKE * 4, dz=FAKE * 3) == 5               # dz over dout
    fc = _dir(FAKE)
    fc.conv_w = FAKE * 7
    assert lib.vm_pool_scan_repeat_bwd(ctypes.byref(fc), None, None, FAKE * 3, 1.0, ctypes.byref(gf), None,
                                       None, 2, 4, 6, 8, 16, 0, 0, 1, None) == 6


def test_conv_bwd_argument_checks(lib):
    def call(x=FAKE, w=FAKE * 2, b=None, du=FAKE * 3, dx=FAKE * 4, dw=FAKE * 5, db=None,
             batch=2, dim=4, L=9, rev=0, dtype=0):
        return lib.vm_causal_conv1d_silu_bwd(x, w, b, du, dx, dw, db, batch, dim, L, rev, dtype, None)

    assert call(x=None) == 1
    assert call(du=None) == 1
    assert call(dx=None) == 1
    assert call(dw=None) == 1
    assert call(L=0) == 2
    assert call(rev=3) == 4
    assert call(dtype=9) == 3
    assert call(dim=1 << 24) == 6                           # one workgroup column per channel
    assert call(dx=FAKE * 3 + 4) == 5                       # dx over du
    assert call(dw=FAKE * 4 + 8) == 5                       # dw over dx
    assert call(db=FAKE * 2) == 5                           # dbias over w
    assert call(b=FAKE * 6, db=FAKE * 6 + 4) == 5           # dbias over bias


def test_row_block_count_limit(lib):
    # scans run one or two 16-channel row blocks per workgroup on grid x: at
    # most 2^24 - 1 row blocks (batch * ceil(dim / 16))
    f, b = _dir(FAKE), _dir(FAKE * 2)
    batch, dim = 1 << 21, 128                               # 2^24 row blocks, L = 1
    assert _scan(lib, batch=batch, dim=dim, L=1) == 6
    assert lib.vm_bidir_scan_fwd(ctypes.byref(f), ctypes.byref(b), None, 1.0, FAKE * 3, batch, dim,
                                 1, 16, 0, 1, None) == 6
    g = vm.VmScanGrad(*(FAKE * 5 + k * (1 << 32) for k in range(7)))
    assert lib.vm_selective_scan_bwd(ctypes.byref(f), None, FAKE * 3, ctypes.byref(g), None, batch,
                                     dim, 1, 16, 0, 1, 0, None) == 6


def test_conv_argument_checks(lib):
    def call(x=FAKE, w=FAKE * 2, b=None, out=FAKE * 3, batch=2, dim=4, L=9, rev=0, dtype=0):
        return lib.vm_causal_conv1d_silu(x, w, b, out, batch, dim, L, rev, dtype, None)

    assert call(x=None) == 1
    assert call(w=None) == 1
    assert call(out=None) == 1
    assert call(L=0) == 2
    assert call(dim=-1) == 2
    assert call(rev=2) == 4
    assert call(dtype=7) == 3
    assert call(batch=1 << 13, dim=1 << 10, L=1 << 10) == 6  # 2^33 elements: 2^23 workgroups
    assert call(out=FAKE + 4) == 5
    assert call(out=FAKE * 2 + 8) == 5                      # overlaps w
    assert call(b=FAKE * 3 + 4) == 5


def test_fused_conv_only_where_supported(lib):
    f, b = _dir(FAKE), _dir(FAKE * 2)
    f.conv_w = FAKE * 5
    # bidirectional: both directions or neither
    assert lib.vm_bidir_scan_fwd(ctypes.byref(f), ctypes.byref(b), None, 1.0, FAKE * 3, 2, 4, 5, 16,
                                 0, 1, None) == 6
    # pooled and SS2D scans take no fused conv
    assert lib.vm_pool_scan_repeat(ctypes.byref(f), None, None, 1.0, FAKE * 3, 2, 4, 2, 2, 16, 0, 0, 1,
                                   None) == 6
    dirs = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 6)) for k in range(4)))
    dirs[1].conv_w = FAKE * 5
    assert lib.vm_ss2d_scan_fwd(dirs, FAKE, None, 1.0, FAKE * 3, 2, 4, 2, 2, 16, 0, 1, None) == 6
    # the conv weights count as inputs for the alias check
    assert _scan(lib, d=f, out=f.conv_w + 4) == 5


def test_bwd_argument_checks(lib):
    f, b = _dir(FAKE), _dir(FAKE * 2)

    def grads(base):
        return vm.VmScanGrad(*(base + k * (1 << 32) for k in range(7)))

    gf, gb = grads(FAKE * 5), grads(FAKE * 6)

    def single(p=f, z=None, dout=FAKE * 3, g=gf, dz=None, N=16, dtype=0, opt=1, rev=0, L=5):
        gp = ctypes.byref(g) if g is not None else None
        return lib.vm_selective_scan_bwd(ctypes.byref(p), z, dout, gp, dz, 2, 4, L, N, dtype, opt, rev, None)

    assert single(dout=None) == 1
    assert single(g=None) == 1
    assert single(z=FAKE * 4) == 1                          # z without dz
    g0 = grads(FAKE * 5)
    g0.dC = None
    assert single(g=g0) == 1
    assert single(dtype=2) == 3
    assert single(opt=3, N=17) == 6                         # zero-order hold accepted, N not
    assert single(dtype=1, opt=3, rev=2) == 4
    assert single(N=17) == 6
    assert single(rev=2) == 4
    assert single(opt=4) == 4
    ga = grads(FAKE * 5)
    ga.du = f.u                                             # a gradient over an input
    assert single(g=ga) == 5
    ga = grads(FAKE * 5)
    ga.dB = ga.dA                                           # gradients over each other
    assert single(g=ga) == 5
    assert single(z=FAKE * 4, dz=FAKE * 3) == 5             # dz over dout
    fc = _dir(FAKE)
    fc.conv_w = FAKE * 7
    assert single(p=fc) == 1                                # fused conv: dconv_w required
    gc = grads(FAKE * 5)
    gc.dconv_w = FAKE + 8                                   # ... and not over an input (u)
    assert single(p=fc, g=gc) == 5

    # token-major B and C with a projection-split stride (44) whose batch-row
    # extent passes the backward kernel's 32-bit byte offsets: rejected
    # before anything runs (L = 13e6: (L + 8) * 44 * 4 bytes > 2^31)
    fs = _dir(FAKE)
    fs.bc_stride = 44
    Lbig = 13_000_000
    assert lib.vm_selective_scan_bwd(ctypes.byref(fs), None, FAKE * 3, ctypes.byref(gf), None, 1, 1, Lbig, 16,
                                     0, 1, 0, None) == 6
    assert lib.vm_bidir_scan_bwd(ctypes.byref(fs), ctypes.byref(fs), None, FAKE * 3, 1.0, ctypes.byref(gf),
                                 ctypes.byref(gb), None, 1, 1, Lbig, 16, 0, 1, None) == 6

    def bidir(g2=gb, scale=1.0, dtype=0):
        return lib.vm_bidir_scan_bwd(ctypes.byref(f), ctypes.byref(b), None, FAKE * 3, scale,
                                     ctypes.byref(gf), ctypes.byref(g2), None, 2, 4, 5, 16, dtype, 1, None)

    assert bidir(scale=float("inf")) == 6
    assert bidir(dtype=5) == 3
    assert bidir(g2=gf) == 5                                # both directions' gradients in one set


def test_ss2d_bwd_argument_checks(lib):
    dirs = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))

    def gsets():
        return (vm.VmScanGrad * 4)(*(vm.VmScanGrad(*(FAKE * (k + 10) + j * (1 << 32) for j in range(7)))
                                     for k in range(4)))

    def call(d=dirs, u=FAKE, z=None, dout=FAKE * 3, scale=1.0, g=None, du=FAKE * 20, dz=None, H=6, W=5,
             N=16, dtype=0, opt=1, conv=False):
        g = gsets() if g is None else g
        return lib.vm_ss2d_scan_bwd(d, u, z, dout, scale, g, du, dz, 2, 4, H, W, N, dtype, opt, None)

    assert call(d=None) == 1
    assert call(u=None) == 1
    assert call(dout=None) == 1
    assert call(du=None) == 1
    assert call(z=FAKE * 21) == 1                           # z without dz
    assert lib.vm_ss2d_scan_bwd(dirs, FAKE, None, FAKE * 3, 1.0, None, FAKE * 20, None, 2, 4, 6, 5, 16, 0,
                                1, None) == 1
    g = gsets()
    g[2].dC = None
    assert call(g=g) == 1
    assert call(H=0) == 2
    assert call(N=17) == 6
    assert call(scale=float("inf")) == 6
    assert call(H=40000, W=40000) == 6
    assert call(dtype=3) == 3
    assert call(opt=8) == 4
    assert call(du=FAKE + 8) == 5                           # du over u
    assert call(du=dirs[3].B) == 5                          # du over a traversal's B
    assert call(z=FAKE * 21, dz=FAKE * 3) == 5              # dz over dout
    assert call(z=FAKE * 21, dz=FAKE * 20 + 4) == 5         # dz over du
    g = gsets()
    g[1].ddelta = FAKE * 20                                 # a traversal's gradient over du
    assert call(g=g) == 5
    g = gsets()
    g[3].dB = g[0].dB                                       # two traversals' gradients in one buffer
    assert call(g=g) == 5
    g = gsets()
    g[2].dD = dirs[2].D                                     # a gradient over an input
    assert call(g=g) == 5
    bad = (vm.VmScanDir * 4)(*(_dir(FAKE * (k + 4)) for k in range(4)))
    bad[1].conv_w = FAKE * 30                               # no fused conv on the 2-D scan
    assert call(d=bad) == 6
