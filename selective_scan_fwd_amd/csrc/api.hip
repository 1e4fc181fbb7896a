// C ABI of the selective-scan library (declared in include/vm_scan.h):
// host-side argument checks, temporary memory from a library-owned
// stream-ordered pool, and kernel dispatch.  Every check runs before any HIP
// call, so a rejected call launches nothing and touches no device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "vm_internal.h"
#include "vm_scan.h"

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxElems = int64_t{1} << 40;
// The map kernels (gather, scatter, pool, repeat, transpose, merge) run one
// 256-thread workgroup per [H, W] plane on grid x: planes * 256 work-items
// must stay below 2^32.
constexpr int64_t kMaxPlanes = (int64_t{1} << 24) - 1;
// The scan kernels run one to two 16-channel row blocks per workgroup of up
// to 256 work-items on grid x; the same bound on the row-block count keeps
// the work-item count below 2^32.
bool row_blocks_ok(int64_t batch, int64_t dim) { return batch * ((dim + 15) / 16) <= kMaxPlanes; }

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
};
Span span(const void *p, int64_t bytes) {
  Span s;
  if (p != nullptr) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + static_cast<uintptr_t>(bytes);
  }
  return s;
}
bool overlaps(Span a, Span b) { return a.lo != 0 && b.lo != 0 && a.lo < b.hi && b.lo < a.hi; }

bool dims_ok(std::initializer_list<int64_t> dims, int64_t *prod) {
  int64_t p = 1;
  for (int64_t d : dims) {
    if (d <= 0 || d > kMaxDim) return false;
    if (p > kMaxElems / d) return false;
    p *= d;
  }
  *prod = p;
  return true;
}

bool flag_ok(int f) { return f == 0 || f == 1; }
bool options_ok(int o) { return (o & ~(VM_DELTA_SOFTPLUS | VM_ZOH)) == 0; }

// Element extent of B or C: dense [batch, dstate, L], or token-major with
// stride bcs (last element at ((batch*L - 1)*bcs + dstate - 1)).
int64_t bc_extent(int64_t batch, int64_t dstate, int64_t L, int64_t bcs) {
  return bcs > 0 ? (batch * L - 1) * bcs + dstate : batch * dstate * L;
}

// Checks of one scan direction.  u_elems / tok_elems: elements of u and of
// delta; L: length of delta, B and C; dim, dstate: parameter shapes.
int check_dir(const vm_scan_dir *p, int64_t u_elems, int64_t tok_elems, int64_t batch, int64_t L,
              int64_t dim, int64_t dstate, int esize, Span out) {
  if (p == nullptr || p->u == nullptr || p->delta == nullptr || p->A == nullptr ||
      p->B == nullptr || p->C == nullptr || p->D == nullptr)
    return VM_ERR_NULL;
  int64_t unused = 0;
  if (p->bc_stride < 0 || (p->bc_stride > 0 && p->bc_stride < dstate)) return VM_ERR_SHAPE;
  if (p->bc_stride > 0 && !dims_ok({batch, L, p->bc_stride}, &unused)) return VM_ERR_SHAPE;
  const int64_t bc = bc_extent(batch, dstate, L, p->bc_stride);
  const Span ins[] = {span(p->u, u_elems * esize), span(p->delta, tok_elems * esize),
                      span(p->A, dim * dstate * 4), span(p->B, bc * esize),
                      span(p->C, bc * esize), span(p->D, dim * 4),
                      span(p->delta_bias, dim * 4), span(p->conv_w, dim * 16),
                      span(p->conv_b, dim * 4)};
  for (const Span &s : ins)
    if (overlaps(s, out)) return VM_ERR_ALIAS;
  return VM_OK;
}

// ---------------------------------------------------------------- workspace
std::mutex g_pool_mu;
std::map<int, hipMemPool_t> g_pools;

hipError_t pool_for_current_device(hipMemPool_t *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  auto it = g_pools.find(dev);
  if (it != g_pools.end()) {
    *out = it->second;
    return hipSuccess;
  }
  hipMemPoolProps props = {};
  props.allocType = hipMemAllocationTypePinned;
  props.handleTypes = hipMemHandleTypeNone;
  props.location.type = hipMemLocationTypeDevice;
  props.location.id = dev;
  hipMemPool_t pool;
  e = hipMemPoolCreate(&pool, &props);
  if (e != hipSuccess) return e;
  uint64_t keep = UINT64_MAX;  // keep freed blocks cached for the next call
  e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
  if (e != hipSuccess) {
    (void)hipMemPoolDestroy(pool);
    return e;
  }
  g_pools[dev] = pool;
  *out = pool;
  return hipSuccess;
}

// Temporary fp32 buffers that live on `stream` for the duration of one call.
// Requests below kChunk bytes are carved, 256-byte aligned, from shared
// chunks of kChunk bytes; larger ones get an allocation of their own.  Each
// pool free costs the host about 5 to 30 microseconds, so a backward call's
// dozen buffers freed one by one took longer on the host than its kernels
// on the GPU.
class Scratch {
 public:
  explicit Scratch(hipStream_t s) : s_(s) {}
  ~Scratch() {
    for (void *p : ptrs_) (void)hipFreeAsync(p, s_);
  }
  void *bytes(int64_t n, int *status) {
    if (*status != VM_OK) return nullptr;
    const size_t need = (static_cast<size_t>(n) + 255) & ~static_cast<size_t>(255);
    if (need >= kChunk) return alloc(need, status);
    if (base_ == nullptr || used_ + need > kChunk) {
      base_ = static_cast<char *>(alloc(kChunk, status));
      used_ = 0;
      if (base_ == nullptr) return nullptr;
    }
    void *p = base_ + used_;
    used_ += need;
    return p;
  }
  float *get(int64_t floats, int *status) { return static_cast<float *>(bytes(floats * 4, status)); }

 private:
  static constexpr size_t kChunk = size_t{64} << 20;
  void *alloc(size_t n, int *status) {
    hipMemPool_t pool;
    void *p = nullptr;
    if (pool_for_current_device(&pool) != hipSuccess ||
        hipMallocFromPoolAsync(&p, n, pool, s_) != hipSuccess) {
      (void)hipGetLastError();
      *status = VM_ERR_ALLOC;
      return nullptr;
    }
    ptrs_.push_back(p);
    return p;
  }
  hipStream_t s_;
  std::vector<void *> ptrs_;
  char *base_ = nullptr;      // the current chunk, and the bytes of it handed out
  size_t used_ = 0;
};

int hip_status(hipError_t e) { return e == hipSuccess ? VM_OK : VM_ERR_HIP; }

// fp32 view of a token tensor: the tensor itself (fp32) or a widened copy.
const float *as_f32(const void *src, int64_t n, bool bf16, Scratch &ws, hipStream_t s,
                    int *status) {
  if (!bf16) return static_cast<const float *>(src);
  float *dst = ws.get(n, status);
  if (*status == VM_OK) *status = hip_status(vmk::launch_to_f32(src, dst, n, s));
  return dst;
}

// Pointers and B/C strides of one direction for the scan kernel, which reads
// dense [batch, dstate, L] and token-major B and C alike.  widen_bc: the
// kernel runs in fp32 on bf16 B and C (pooled path), so they are widened into
// temporary memory with the same layout first.
vmk::DirPtrs dir_ptrs(const vm_scan_dir *p, int64_t dstate, int64_t L) {
  vmk::DirPtrs d = {};
  d.u = p->u;
  d.delta = p->delta;
  d.A = p->A;
  d.D = p->D;
  d.bias = p->delta_bias;
  d.B = p->B;
  d.C = p->C;
  d.cw = p->conv_w;
  d.cb = p->conv_b;
  if (p->bc_stride > 0) {
    d.bsb = L * p->bc_stride;
    d.bsn = 1;
    d.bst = p->bc_stride;
  } else {
    d.bsb = dstate * L;
    d.bsn = L;
    d.bst = 1;
  }
  return d;
}

vmk::DirPtrs resolve_dir(const vm_scan_dir *p, int64_t batch, int64_t dstate, int64_t L,
                         bool widen_bc, Scratch &ws, hipStream_t s, int *status) {
  vmk::DirPtrs d = dir_ptrs(p, dstate, L);
  if (widen_bc) {
    const int64_t n = bc_extent(batch, dstate, L, p->bc_stride);
    d.B = as_f32(p->B, n, true, ws, s, status);
    d.C = as_f32(p->C, n, true, ws, s, status);
  }
  return d;
}

// Exchange rows of a long bidirectional scan (global exchange): fp32 output
// with line-aligned rows doubles as the exchange buffer; otherwise it comes
// from the pool.  Short scans need none.
int exchange_for(vmk::ScanArgs &a, bool bf16, Scratch &ws) {
  const vmk::ScanPlan plan = vmk::plan_scan(a.batch, a.dim, a.L, a.dstate, 2, a.conv != 0);
  if (plan.xmode != vmk::kXGlobal) return VM_OK;
  int st = VM_OK;
  a.xstride = vmk::xchg_global_stride(a.L);
  if (!bf16 && a.xstride == a.L && reinterpret_cast<uintptr_t>(a.out) % 128 == 0)
    a.xglobal = static_cast<float *>(a.out);
  else
    a.xglobal = ws.get(a.batch * a.dim * a.xstride, &st);
  return st;
}

// Plans and launches a bidirectional scan whose arguments are filled in,
// taking its exchange rows (exchange_for) unless the caller already has.
int launch_bidir(vmk::ScanArgs &a, bool bf16, Scratch &ws, hipStream_t s) {
  const vmk::ScanPlan plan = vmk::plan_scan(a.batch, a.dim, a.L, a.dstate, 2, a.conv != 0);
  int st = VM_OK;
  if (plan.xmode == vmk::kXGlobal && a.xglobal == nullptr) {
    st = exchange_for(a, bf16, ws);
    if (st != VM_OK) return st;
  }
  if (!vmk::scan_offsets_fit(plan, a, bf16)) return VM_ERR_UNSUPPORTED;
  return hip_status(vmk::launch_scan(plan, a, bf16, s));
}

// Temporary memory and launches of one direction's backward pass after dy
// is known: the kernel, then the reduction of its partial sums into g.
struct BwdScratch {
  float *ck = nullptr, *pA = nullptr, *pD = nullptr, *pbias = nullptr, *pB = nullptr, *pC = nullptr;
  int get(Scratch &ws, int64_t batch, int64_t dim, int64_t L) {
    int st = VM_OK;
    ck = ws.get(vmk::scan_bwd_ck_floats(batch, dim, L), &st);
    pA = ws.get(batch * dim * 16, &st);
    pD = ws.get(batch * dim, &st);
    pbias = ws.get(batch * dim, &st);
    pB = ws.get(vmk::scan_bwd_tiled_floats(batch, dim, L), &st);
    pC = ws.get(vmk::scan_bwd_tiled_floats(batch, dim, L), &st);
    return st;
  }
};

// How a backward pass finds what its forward recomputation prepared.
enum class Prep { kNone, kCk, kCkDyTiled };

vmk::BwdArgs bwd_args(const vm_scan_dir *p, const float *dy, const vm_scan_grad *g, const BwdScratch &bs,
                      int64_t batch, int64_t dim, int64_t L, int64_t dstate, int options, int reverse,
                      Prep prep, Scratch &ws, hipStream_t s, int *st) {
  vmk::BwdArgs a = {};
  // checkpoints from the forward kernel; with the gate's backward fused
  // there, dy is tile-major too
  a.ck_ready = prep != Prep::kNone ? 1 : 0;
  a.dy_tiled = prep == Prep::kCkDyTiled ? 1 : 0;
  a.dir = resolve_dir(p, batch, dstate, L, false, ws, s, st);
  a.dy = dy;
  a.du = g->du;
  a.ddelta = g->ddelta;
  a.ck = bs.ck;
  a.pA = bs.pA;
  a.pD = bs.pD;
  a.pbias = bs.pbias;
  a.pB = bs.pB;
  a.pC = bs.pC;
  a.batch = batch;
  a.dim = dim;
  a.L = L;
  a.dstate = static_cast<int>(dstate);
  a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
  a.zoh = (options & VM_ZOH) != 0;
  a.reverse = reverse;
  return a;
}

// n (<= 4) directions' backward passes of one shape: one launch of the
// kernel over all of them (more waves in flight than one direction's), then
// each direction's reductions.  bs[k] holds direction k's checkpoints and
// partial sums.
int run_bwd_group(int n, const vm_scan_dir *const p[], const float *const dy[], const vm_scan_grad *const g[],
                  const BwdScratch bs[], int64_t batch, int64_t dim, int64_t L, int64_t dstate, int options,
                  const int reverse[], Scratch &ws, hipStream_t s, Prep prep = Prep::kNone) {
  int st = VM_OK;
  vmk::BwdGroup grp = {};
  grp.n = n;
  for (int k = 0; k < n; ++k)
    grp.a[k] = bwd_args(p[k], dy[k], g[k], bs[k], batch, dim, L, dstate, options, reverse[k], prep, ws, s,
                        &st);
  if (st != VM_OK) return st;
  st = hip_status(vmk::launch_scan_bwd_group(grp, s));
  vmk::BwdReduceOut out[vmk::kBwdGroupMax] = {};
  for (int k = 0; k < n; ++k) out[k] = {g[k]->dA, g[k]->dB, g[k]->dC, g[k]->dD, g[k]->ddelta_bias};
  if (st == VM_OK) st = hip_status(vmk::launch_scan_bwd_reduce_group(grp, out, s));
  return st;
}

int run_bwd(const vm_scan_dir *p, const float *dy, const vm_scan_grad *g, const BwdScratch &bs,
            int64_t batch, int64_t dim, int64_t L, int64_t dstate, int options, int reverse,
            Scratch &ws, hipStream_t s, Prep prep = Prep::kNone) {
  return run_bwd_group(1, &p, &dy, &g, &bs, batch, dim, L, dstate, options, &reverse, ws, s, prep);
}

// Checks of a gradient set: required pointers, no overlap with the inputs
// (ins) or with the other outputs (outs, extended here).
int check_grad(const vm_scan_grad *g, int64_t tok, int64_t bc, int64_t dim, int64_t dstate,
               bool conv, const std::vector<Span> &ins, std::vector<Span> &outs,
               int64_t tok_u = -1, bool need_du = true) {
  if (tok_u < 0) tok_u = tok;       // elements of du (full resolution on the pooled path)
  if (g == nullptr || (need_du && g->du == nullptr) || g->ddelta == nullptr || g->dA == nullptr ||
      g->dB == nullptr || g->dC == nullptr || g->dD == nullptr || (conv && g->dconv_w == nullptr))
    return VM_ERR_NULL;
  const Span mine[] = {span(g->du, tok_u * 4), span(g->ddelta, tok * 4), span(g->dA, dim * dstate * 4),
                       span(g->dB, bc * 4), span(g->dC, bc * 4), span(g->dD, dim * 4),
                       span(g->ddelta_bias, dim * 4),
                       conv ? span(g->dconv_w, dim * 16) : Span(),
                       conv ? span(g->dconv_b, dim * 4) : Span()};
  for (const Span &m : mine) {
    for (const Span &i : ins)
      if (overlaps(m, i)) return VM_ERR_ALIAS;
    for (const Span &o : outs)
      if (overlaps(m, o)) return VM_ERR_ALIAS;
    outs.push_back(m);
  }
  return VM_OK;
}

void dir_spans(const vm_scan_dir *p, int64_t tok, int64_t batch, int64_t L, int64_t dim,
               int64_t dstate, int es, std::vector<Span> &ins) {
  const int64_t bc = bc_extent(batch, dstate, L, p->bc_stride);
  const Span sp[] = {span(p->u, tok * es), span(p->delta, tok * es), span(p->A, dim * dstate * 4),
                     span(p->B, bc * es), span(p->C, bc * es), span(p->D, dim * 4),
                     span(p->delta_bias, dim * 4), span(p->conv_w, dim * 16),
                     span(p->conv_b, dim * 4)};
  ins.insert(ins.end(), sp, sp + 9);
}

// fp32 view of a direction's token tensors for the backward pass: the
// direction itself, or (bf16) one whose u, delta, B and C are widened copies
// in the same layout.
vm_scan_dir widen_dir(const vm_scan_dir *p, int64_t tok, int64_t batch, int64_t L,
                      int64_t dstate, bool bf16, Scratch &ws, hipStream_t s, int *st) {
  vm_scan_dir w = *p;
  if (!bf16) return w;
  const int64_t bc = bc_extent(batch, dstate, L, p->bc_stride);
  w.u = as_f32(p->u, tok, true, ws, s, st);
  w.delta = as_f32(p->delta, tok, true, ws, s, st);
  w.B = as_f32(p->B, bc, true, ws, s, st);
  w.C = as_f32(p->C, bc, true, ws, s, st);
  return w;
}

// The fused conv around a direction's backward: its input x (fp32), the
// conv output u it scans (temporary), and the temporary u gradient, which the
// conv backward turns into the x, weight and bias gradients of g.
struct ConvBwd {
  const float *x = nullptr;
  float *u = nullptr, *du = nullptr, *partial = nullptr;
  int get(Scratch &ws, int64_t tok, int64_t batch, int64_t dim) {
    int st = VM_OK, rpc = 0;
    u = ws.get(tok, &st);
    du = ws.get(tok, &st);
    partial = ws.get(static_cast<int64_t>(vmk::conv1d_bwd_chunks(batch, dim, &rpc)) * dim * 5, &st);
    return st;
  }
  // u = SiLU(conv(x)); the direction then scans u without the conv
  int forward(vm_scan_dir &w, int64_t batch, int64_t dim, int64_t L, int reverse, hipStream_t s) {
    x = static_cast<const float *>(w.u);
    const int st = hip_status(vmk::launch_conv1d_silu(x, w.conv_w, w.conv_b, u, batch * dim, L, dim,
                                                      reverse, false, s));
    w.u = u;
    return st;
  }
  int backward(const vm_scan_dir &p, const vm_scan_grad *g, int64_t batch, int64_t dim, int64_t L,
               int reverse, hipStream_t s) {
    return hip_status(vmk::launch_conv1d_silu_bwd(x, p.conv_w, p.conv_b, du, g->du, g->dconv_w,
                                                  g->dconv_b, partial, batch, dim, L, reverse,
                                                  false, s));
  }
};

// Shared checks of the backward entry points (dz exactly when z).
// The backward kernel reads one batch row of B and C (fp32, after any
// widening, which keeps the layout) through a buffer resource with 32-bit
// byte offsets, up to one tile past the last step: reject layouts whose
// extent would not fit.
int check_bwd_bc(const vm_scan_dir *p, int64_t L, int64_t dstate) {
  if (p == nullptr) return VM_OK;
  const int64_t bsn = p->bc_stride > 0 ? 1 : L;
  const int64_t bst = p->bc_stride > 0 ? p->bc_stride : 1;
  const int64_t ext = (dstate - 1) * bsn + (L + vmk::kBwdTile) * bst + 1;
  return ext * 4 < (int64_t{1} << 31) ? VM_OK : VM_ERR_UNSUPPORTED;
}

int check_bwd_common(int dtype, int options, int64_t batch, int64_t dim, int64_t L, int64_t dstate,
                     const void *z, const void *dout, const void *dz, int64_t *tok, int64_t *bc) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!options_ok(options)) return VM_ERR_FLAG;
  if (!dims_ok({batch, dim, L}, tok) || dstate <= 0) return VM_ERR_SHAPE;
  // (the parameter-gradient reduction runs one workgroup per channel)
  if (dstate > 16 || dim > kMaxPlanes || !row_blocks_ok(batch, dim)) return VM_ERR_UNSUPPORTED;
  if (!dims_ok({batch, dstate, L}, bc)) return VM_ERR_SHAPE;
  // 32-bit offsets of the kernel's per-block checkpoints and partial sums
  if (16 * 64 * vmk::scan_bwd_tiles(L) >= (int64_t{1} << 31) || 64 * L >= (int64_t{1} << 31))
    return VM_ERR_UNSUPPORTED;
  if (dout == nullptr || (z != nullptr && dz == nullptr)) return VM_ERR_NULL;
  return VM_OK;
}

}  // namespace

extern "C" {

const char *vm_status_string(int status) {
  switch (status) {
    case VM_OK: return "VM_OK";
    case VM_ERR_NULL: return "VM_ERR_NULL: a required pointer is NULL";
    case VM_ERR_SHAPE: return "VM_ERR_SHAPE: a size is <= 0 or an element count overflows";
    case VM_ERR_DTYPE: return "VM_ERR_DTYPE: unknown dtype";
    case VM_ERR_FLAG: return "VM_ERR_FLAG: a flag is not 0 or 1, or unknown option bits";
    case VM_ERR_ALIAS: return "VM_ERR_ALIAS: the output overlaps an input";
    case VM_ERR_UNSUPPORTED: return "VM_ERR_UNSUPPORTED: dstate outside [1, 16], non-finite scale, or sizes past the kernels' 32-bit offsets or grid limits";
    case VM_ERR_HIP: return "VM_ERR_HIP: a HIP launch or runtime call failed";
    case VM_ERR_ALLOC: return "VM_ERR_ALLOC: temporary device memory unavailable";
    default: return "unknown status";
  }
}

int vm_version(void) { return 10000; }

int64_t vm_atrous_group_len(int64_t height, int64_t width) {
  if (height <= 0 || width <= 0 || height > kMaxDim || width > kMaxDim) return -VM_ERR_SHAPE;
  return ((height + 1) / 2) * ((width + 1) / 2);
}

int vm_selective_scan_fwd(const vm_scan_dir *p, const void *z, void *out, int64_t batch,
                          int64_t dim, int64_t seqlen, int64_t dstate, int dtype,
                          int options, int reverse, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!options_ok(options) || !flag_ok(reverse)) return VM_ERR_FLAG;
  int64_t tok = 0, bc = 0;
  if (!dims_ok({batch, dim, seqlen}, &tok) || dstate <= 0) return VM_ERR_SHAPE;
  if (dstate > 16 || !row_blocks_ok(batch, dim)) return VM_ERR_UNSUPPORTED;
  if (!dims_ok({batch, dstate, seqlen}, &bc)) return VM_ERR_SHAPE;
  if (out == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span so = span(out, tok * es);
  int st = check_dir(p, tok, tok, batch, seqlen, dim, dstate, es, so);
  if (st != VM_OK) return st;
  if (overlaps(span(z, tok * es), so)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == VM_BF16;
  Scratch ws(s);
  vmk::ScanArgs a = {};
  a.dir[0] = a.dir[1] = resolve_dir(p, batch, dstate, seqlen, false, ws, s, &st);
  if (st != VM_OK) return st;
  a.z = z;
  a.out = out;
  a.batch = batch;
  a.dim = dim;
  a.L = seqlen;
  a.dstate = static_cast<int>(dstate);
  a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
  a.zoh = (options & VM_ZOH) != 0;
  a.reverse = reverse;
  a.scale = 1.0f;
  a.conv = p->conv_w != nullptr;
  const vmk::ScanPlan plan = vmk::plan_scan(batch, dim, seqlen, a.dstate, 1, a.conv != 0);
  if (!vmk::scan_offsets_fit(plan, a, bf16)) return VM_ERR_UNSUPPORTED;
  return hip_status(vmk::launch_scan(plan, a, bf16, s));
}

}  // extern "C"

namespace {

// Host-side checks of the bidirectional forward entry points, and the
// kernel arguments of a call that passes them (everything but the exchange).
int bidir_fwd_args(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z, float combine_scale,
                   void *out, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int dtype,
                   int options, vmk::ScanArgs *a) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!options_ok(options)) return VM_ERR_FLAG;
  int64_t tok = 0, bc = 0;
  if (!dims_ok({batch, dim, seqlen}, &tok) || dstate <= 0) return VM_ERR_SHAPE;
  if (dstate > 16 || !std::isfinite(combine_scale) || !row_blocks_ok(batch, dim))
    return VM_ERR_UNSUPPORTED;
  if (!dims_ok({batch, dstate, seqlen}, &bc)) return VM_ERR_SHAPE;
  if (out == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span so = span(out, tok * es);
  int st = check_dir(fwd, tok, tok, batch, seqlen, dim, dstate, es, so);
  if (st == VM_OK) st = check_dir(bwd, tok, tok, batch, seqlen, dim, dstate, es, so);
  if (st != VM_OK) return st;
  if ((fwd->conv_w == nullptr) != (bwd->conv_w == nullptr)) return VM_ERR_UNSUPPORTED;
  if (overlaps(span(z, tok * es), so)) return VM_ERR_ALIAS;
  *a = vmk::ScanArgs{};
  a->dir[0] = dir_ptrs(fwd, dstate, seqlen);
  a->dir[1] = dir_ptrs(bwd, dstate, seqlen);
  a->z = z;
  a->out = out;
  a->batch = batch;
  a->dim = dim;
  a->L = seqlen;
  a->dstate = static_cast<int>(dstate);
  a->softplus = (options & VM_DELTA_SOFTPLUS) != 0;
  a->zoh = (options & VM_ZOH) != 0;
  a->reverse = 0;
  a->scale = combine_scale;
  a->conv = fwd->conv_w != nullptr;
  return VM_OK;
}

// ---- the exchange buffer of vm_bidir_scan_fwd_noalloc, for callers that
// cannot allocate: a file-scope device array of kNoAllocFloats fp32 values
// (32 MiB), one copy per GPU the library runs on, held until the process
// ends.  Host code never passes the array's name to a kernel: it takes the
// device address once per device with hipGetSymbolAddress and uses that.
constexpr int64_t kNoAllocFloats = int64_t{8} << 20;
static __device__ __align__(256) float scratch[kNoAllocFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(float **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return VM_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return VM_ERR_HIP;
    }
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  *out = g_scratch_ptr[dev];
  return VM_OK;
}

}  // namespace

extern "C" {

int vm_bidir_scan_fwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z,
                      float combine_scale, void *out, int64_t batch, int64_t dim,
                      int64_t seqlen, int64_t dstate, int dtype, int options,
                      void *stream) {
  vmk::ScanArgs a;
  int st = bidir_fwd_args(fwd, bwd, z, combine_scale, out, batch, dim, seqlen, dstate, dtype, options, &a);
  if (st != VM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  return launch_bidir(a, dtype == VM_BF16, ws, s);
}

int vm_bidir_scan_fwd_noalloc(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z,
                              float combine_scale, void *out, int64_t batch, int64_t dim,
                              int64_t seqlen, int64_t dstate, int dtype, int options,
                              void *stream) {
  vmk::ScanArgs a;
  int st = bidir_fwd_args(fwd, bwd, z, combine_scale, out, batch, dim, seqlen, dstate, dtype, options, &a);
  if (st != VM_OK) return st;
  const bool bf16 = dtype == VM_BF16;
  const vmk::ScanPlan plan = vmk::plan_scan(batch, dim, seqlen, static_cast<int>(dstate), 2, a.conv != 0);
  if (plan.xmode == vmk::kXGlobal) {
    a.xstride = vmk::xchg_global_stride(seqlen);
    if (!bf16 && a.xstride == seqlen && reinterpret_cast<uintptr_t>(out) % 128 == 0) {
      a.xglobal = static_cast<float *>(out);        // out serves as the exchange, as in vm_bidir_scan_fwd
    } else {
      if (batch * dim > kNoAllocFloats / a.xstride) return VM_ERR_UNSUPPORTED;
      st = scratch_on_current_device(&a.xglobal);
      if (st != VM_OK) return st;
    }
  }
  if (!vmk::scan_offsets_fit(plan, a, bf16)) return VM_ERR_UNSUPPORTED;
  return hip_status(vmk::launch_scan(plan, a, bf16, static_cast<hipStream_t>(stream)));
}

int vm_causal_conv1d_silu(const void *x, const float *w, const float *bias, void *out,
                          int64_t batch, int64_t dim, int64_t seqlen, int reverse, int dtype,
                          void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!flag_ok(reverse)) return VM_ERR_FLAG;
  int64_t tok = 0;
  if (!dims_ok({batch, dim, seqlen}, &tok)) return VM_ERR_SHAPE;
  // one 256-thread workgroup per 2048 consecutive elements on grid x, whose
  // work-item count must stay below 2^32
  if (tok >= (int64_t{1} << 33)) return VM_ERR_UNSUPPORTED;
  if (x == nullptr || w == nullptr || out == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span so = span(out, tok * es);
  if (overlaps(span(x, tok * es), so) || overlaps(span(w, dim * 16), so) ||
      overlaps(span(bias, dim * 4), so))
    return VM_ERR_ALIAS;
  return hip_status(vmk::launch_conv1d_silu(x, w, bias, out, batch * dim, seqlen, dim, reverse,
                                            dtype == VM_BF16, static_cast<hipStream_t>(stream)));
}

int vm_causal_conv1d_silu_bwd(const void *x, const float *w, const float *bias, const float *du,
                              float *dx, float *dw, float *dbias, int64_t batch, int64_t dim,
                              int64_t seqlen, int reverse, int dtype, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!flag_ok(reverse)) return VM_ERR_FLAG;
  int64_t tok = 0;
  if (!dims_ok({batch, dim, seqlen}, &tok)) return VM_ERR_SHAPE;
  // one workgroup per (channel, chunk of batch rows): dim on grid x, a
  // chunk's elements counted in 32 bits
  int rpc = 0;
  vmk::conv1d_bwd_chunks(batch, dim, &rpc);
  if (dim > kMaxPlanes || static_cast<int64_t>(rpc) * seqlen >= (int64_t{1} << 31))
    return VM_ERR_UNSUPPORTED;
  if (x == nullptr || w == nullptr || du == nullptr || dx == nullptr || dw == nullptr)
    return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span ins[] = {span(x, tok * es), span(w, dim * 16), span(bias, dim * 4), span(du, tok * 4)};
  const Span outs[] = {span(dx, tok * 4), span(dw, dim * 16), span(dbias, dim * 4)};
  for (int o = 0; o < 3; ++o) {
    for (const Span &i : ins)
      if (overlaps(outs[o], i)) return VM_ERR_ALIAS;
    for (int o2 = 0; o2 < o; ++o2)
      if (overlaps(outs[o], outs[o2])) return VM_ERR_ALIAS;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  int st = VM_OK;
  const int nchunk = vmk::conv1d_bwd_chunks(batch, dim, &rpc);
  float *partial = ws.get(static_cast<int64_t>(nchunk) * dim * 5, &st);
  if (st != VM_OK) return st;
  return hip_status(vmk::launch_conv1d_silu_bwd(x, w, bias, du, dx, dw, dbias, partial, batch, dim,
                                                seqlen, reverse, dtype == VM_BF16, s));
}

int vm_atrous_gather(const void *x, void *streams, int64_t batch, int64_t channels,
                     int64_t height, int64_t width, int dtype, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  int64_t n_in = 0, n_out = 0;
  const int64_t Lg = vm_atrous_group_len(height, width);
  if (Lg <= 0 || !dims_ok({batch, channels, height, width}, &n_in) ||
      !dims_ok({batch, 4, channels, Lg}, &n_out))
    return VM_ERR_SHAPE;
  if (batch * channels > kMaxPlanes) return VM_ERR_UNSUPPORTED;
  if (x == nullptr || streams == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  if (overlaps(span(x, n_in * es), span(streams, n_out * es))) return VM_ERR_ALIAS;
  return hip_status(vmk::launch_atrous_gather(x, streams, batch, channels, height, width,
                                              dtype == VM_BF16, static_cast<hipStream_t>(stream)));
}

int vm_atrous_scatter(const void *streams, void *y, int64_t batch, int64_t channels,
                      int64_t height, int64_t width, int dtype, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  int64_t n_out = 0, n_in = 0;
  const int64_t Lg = vm_atrous_group_len(height, width);
  if (Lg <= 0 || !dims_ok({batch, channels, height, width}, &n_out) ||
      !dims_ok({batch, 4, channels, Lg}, &n_in))
    return VM_ERR_SHAPE;
  if (batch * channels > kMaxPlanes) return VM_ERR_UNSUPPORTED;
  if (streams == nullptr || y == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  if (overlaps(span(streams, n_in * es), span(y, n_out * es))) return VM_ERR_ALIAS;
  return hip_status(vmk::launch_atrous_scatter(streams, y, batch, channels, height, width,
                                               dtype == VM_BF16, static_cast<hipStream_t>(stream)));
}

int vm_pool_scan_repeat(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z,
                        float combine_scale, void *out, int64_t batch, int64_t dim,
                        int64_t height, int64_t width, int64_t dstate, int pool_axis,
                        int dtype, int options, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!options_ok(options) || !flag_ok(pool_axis)) return VM_ERR_FLAG;
  const int64_t Lp = pool_axis == 0 ? height : width;
  int64_t full = 0, pooled = 0, bc = 0;
  if (!dims_ok({batch, dim, height, width}, &full) || !dims_ok({batch, dim, Lp}, &pooled) ||
      dstate <= 0)
    return VM_ERR_SHAPE;
  if (dstate > 16 || !std::isfinite(combine_scale) || batch * dim > kMaxPlanes)
    return VM_ERR_UNSUPPORTED;
  if (!dims_ok({batch, dstate, Lp}, &bc)) return VM_ERR_SHAPE;
  if (out == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span so = span(out, full * es);
  int st = check_dir(fwd, full, pooled, batch, Lp, dim, dstate, es, so);
  if (st == VM_OK && bwd != nullptr) st = check_dir(bwd, full, pooled, batch, Lp, dim, dstate, es, so);
  if (st != VM_OK) return st;
  if (fwd->conv_w != nullptr || (bwd != nullptr && bwd->conv_w != nullptr)) return VM_ERR_UNSUPPORTED;
  if (overlaps(span(z, full * es), so)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == VM_BF16;
  const int ndir = bwd != nullptr ? 2 : 1;
  const vm_scan_dir *dirs[2] = {fwd, bwd};
  Scratch ws(s);
  float *y = ws.get(pooled, &st);
  vmk::ScanArgs a = {};
  for (int k = 0; k < ndir; ++k) {
    const vm_scan_dir *p = dirs[k];
    float *ubar = ws.get(pooled, &st);
    if (st != VM_OK) return st;
    st = hip_status(vmk::launch_mean_pool(p->u, ubar, batch * dim, height, width, pool_axis,
                                          bf16, s));
    const float *dl = as_f32(p->delta, pooled, bf16, ws, s, &st);
    vmk::DirPtrs d = resolve_dir(p, batch, dstate, Lp, bf16, ws, s, &st);
    if (st != VM_OK) return st;
    d.u = ubar;
    d.delta = dl;
    a.dir[k] = d;
  }
  if (ndir == 1) a.dir[1] = a.dir[0];
  a.z = nullptr;
  a.out = y;
  a.batch = batch;
  a.dim = dim;
  a.L = Lp;
  a.dstate = static_cast<int>(dstate);
  a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
  a.zoh = (options & VM_ZOH) != 0;
  a.reverse = 0;
  a.scale = 1.0f;
  const vmk::ScanPlan plan = vmk::plan_scan(batch, dim, Lp, a.dstate, ndir, false);
  if (plan.xmode == vmk::kXGlobal) {
    a.xstride = vmk::xchg_global_stride(Lp);
    a.xglobal = ws.get(batch * dim * a.xstride, &st);
    if (st != VM_OK) return st;
  }
  if (!vmk::scan_offsets_fit(plan, a, /*bf16=*/false)) return VM_ERR_UNSUPPORTED;
  st = hip_status(vmk::launch_scan(plan, a, /*bf16=*/false, s));
  if (st != VM_OK) return st;
  return hip_status(vmk::launch_repeat_gate(y, z, out, batch * dim, height, width, pool_axis,
                                            combine_scale, bf16, s));
}

int vm_pool_scan_repeat_bwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z,
                            const void *dout, float combine_scale, const vm_scan_grad *gf,
                            const vm_scan_grad *gb, void *dz, int64_t batch, int64_t dim,
                            int64_t height, int64_t width, int64_t dstate, int pool_axis, int dtype,
                            int options, void *stream) {
  if (!flag_ok(pool_axis)) return VM_ERR_FLAG;
  const int64_t Lp = pool_axis == 0 ? height : width;
  int64_t full = 0, pooled = 0, bc = 0;
  if (!dims_ok({batch, dim, height, width}, &full)) return VM_ERR_SHAPE;
  int st = check_bwd_common(dtype, options, batch, dim, Lp, dstate, z, dout, dz, &pooled, &bc);
  if (st != VM_OK) return st;
  if (!std::isfinite(combine_scale) || batch * dim > kMaxPlanes) return VM_ERR_UNSUPPORTED;
  const bool bf16 = dtype == VM_BF16;
  const int es = bf16 ? 2 : 4;
  st = check_dir(fwd, full, pooled, batch, Lp, dim, dstate, es, Span());
  if (st == VM_OK && bwd != nullptr) st = check_dir(bwd, full, pooled, batch, Lp, dim, dstate, es, Span());
  if (st == VM_OK) st = check_bwd_bc(fwd, Lp, dstate);
  if (st == VM_OK) st = check_bwd_bc(bwd, Lp, dstate);
  if (st != VM_OK) return st;
  if (fwd->conv_w != nullptr || (bwd != nullptr && bwd->conv_w != nullptr)) return VM_ERR_UNSUPPORTED;
  const int ndir = bwd != nullptr ? 2 : 1;
  const vm_scan_dir *dirs[2] = {fwd, bwd};
  const vm_scan_grad *grads[2] = {gf, gb};
  std::vector<Span> ins, outs;
  for (int k = 0; k < ndir; ++k) {
    dir_spans(dirs[k], pooled, batch, Lp, dim, dstate, es, ins);
    ins.push_back(span(dirs[k]->u, full * es));     // u is full resolution here
  }
  ins.push_back(span(z, full * es));
  ins.push_back(span(dout, full * es));
  for (int k = 0; k < ndir && st == VM_OK; ++k)
    st = check_grad(grads[k], pooled, bc, dim, dstate, false, ins, outs, full);
  if (st != VM_OK) return st;
  for (const Span &o : outs)
    if (overlaps(span(dz, full * 4), o)) return VM_ERR_ALIAS;
  for (const Span &i : ins)
    if (overlaps(span(dz, full * 4), i)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  // temporary memory first: pooled u per direction, the pooled forward
  // output and its gradient, the scans' u gradient, the backward scratch
  float *ubar[2] = {nullptr, nullptr};
  for (int k = 0; k < ndir; ++k) ubar[k] = ws.get(pooled, &st);
  float *y = ws.get(pooled, &st);
  float *dyp = ws.get(pooled, &st);
  float *dubar = ws.get(pooled, &st);
  BwdScratch bs;
  if (st == VM_OK) st = bs.get(ws, batch, dim, Lp);
  vmk::ScanArgs a = {};                 // the pooled forward scan (ungated, scale 1)
  a.out = y;
  a.batch = batch;
  a.dim = dim;
  a.L = Lp;
  a.dstate = static_cast<int>(dstate);
  if (st == VM_OK && ndir == 2) st = exchange_for(a, false, ws);
  if (st != VM_OK) return st;
  // the directions as the pooled scans see them (fp32)
  vm_scan_dir w[2];
  for (int k = 0; k < ndir; ++k) {
    w[k] = *dirs[k];
    st = hip_status(vmk::launch_mean_pool(dirs[k]->u, ubar[k], batch * dim, height, width, pool_axis,
                                          bf16, s));
    if (st != VM_OK) return st;
    w[k].u = ubar[k];
    w[k].delta = as_f32(dirs[k]->delta, pooled, bf16, ws, s, &st);
    if (bf16) {
      const int64_t n = bc_extent(batch, dstate, Lp, dirs[k]->bc_stride);
      w[k].B = as_f32(dirs[k]->B, n, true, ws, s, &st);
      w[k].C = as_f32(dirs[k]->C, n, true, ws, s, &st);
    }
    if (st != VM_OK) return st;
    a.dir[k] = resolve_dir(&w[k], batch, dstate, Lp, false, ws, s, &st);
  }
  if (ndir == 1) a.dir[1] = a.dir[0];
  if (st != VM_OK) return st;
  a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
  a.zoh = (options & VM_ZOH) != 0;
  a.scale = 1.0f;
  if (ndir == 2) {
    st = launch_bidir(a, false, ws, s);
  } else {
    const vmk::ScanPlan plan = vmk::plan_scan(batch, dim, Lp, a.dstate, 1, false);
    if (!vmk::scan_offsets_fit(plan, a, false)) return VM_ERR_UNSUPPORTED;
    st = hip_status(vmk::launch_scan(plan, a, false, s));
  }
  if (st != VM_OK) return st;
  // gate and repeat backward: dz, and the pooled output's gradient
  st = hip_status(vmk::launch_repeat_gate_bwd(y, z, dout, dyp, static_cast<float *>(dz), batch * dim,
                                              height, width, pool_axis, combine_scale, bf16, s));
  for (int k = 0; k < ndir && st == VM_OK; ++k) {
    vm_scan_grad gu = *grads[k];
    gu.du = dubar;
    st = run_bwd(&w[k], dyp, &gu, bs, batch, dim, Lp, dstate, options, k, ws, s);
    if (st == VM_OK)
      st = hip_status(vmk::launch_pool_bwd(dubar, grads[k]->du, batch * dim, height, width, pool_axis, s));
  }
  return st;
}

int vm_ss2d_scan_fwd(const vm_scan_dir *dirs, const void *u, const void *z, float combine_scale,
                     void *out, int64_t batch, int64_t dim, int64_t height, int64_t width,
                     int64_t dstate, int dtype, int options, void *stream) {
  if (dtype != VM_F32 && dtype != VM_BF16) return VM_ERR_DTYPE;
  if (!options_ok(options)) return VM_ERR_FLAG;
  int64_t tok = 0, bc = 0;
  if (!dims_ok({batch, dim, height, width}, &tok) || dstate <= 0) return VM_ERR_SHAPE;
  const int64_t L = height * width;
  if (dstate > 16 || !std::isfinite(combine_scale) || batch * dim > kMaxPlanes)
    return VM_ERR_UNSUPPORTED;
  if (!dims_ok({batch, dstate, L}, &bc)) return VM_ERR_SHAPE;
  // merge / transpose grids: 32 x 32 tiles of one map on grid y
  if (((height + 31) / 32) * ((width + 31) / 32) > 65535) return VM_ERR_UNSUPPORTED;
  if (dirs == nullptr || u == nullptr || out == nullptr) return VM_ERR_NULL;
  const int es = dtype == VM_BF16 ? 2 : 4;
  const Span so = span(out, tok * es);
  vm_scan_dir d[4];
  int st = VM_OK;
  for (int k = 0; k < 4 && st == VM_OK; ++k) {
    d[k] = dirs[k];
    d[k].u = u;                     // the one map every traversal reads
    st = check_dir(&d[k], tok, tok, batch, L, dim, dstate, es, so);
    if (st == VM_OK && d[k].conv_w != nullptr) st = VM_ERR_UNSUPPORTED;
  }
  if (st != VM_OK) return st;
  if (overlaps(span(z, tok * es), so)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == VM_BF16;
  Scratch ws(s);
  // The scans run in fp32: bf16 inputs are widened first.  Rows (traversals
  // 0, 1) scan u as it is; columns (2, 3) scan its transpose.
  const float *u32 = as_f32(u, tok, bf16, ws, s, &st);
  float *ut = ws.get(tok, &st);
  float *yc = ws.get(tok, &st);
  float *yr = bf16 ? ws.get(tok, &st) : static_cast<float *>(out);
  if (st != VM_OK) return st;
  st = hip_status(vmk::launch_transpose(u32, ut, batch * dim, height, width, false, s));
  for (int pass = 0; pass < 2 && st == VM_OK; ++pass) {
    vmk::ScanArgs a = {};
    for (int k = 0; k < 2; ++k) {
      const vm_scan_dir *p = &d[2 * pass + k];
      vmk::DirPtrs dp = resolve_dir(p, batch, dstate, L, bf16, ws, s, &st);
      dp.u = pass == 0 ? u32 : ut;
      dp.delta = as_f32(p->delta, tok, bf16, ws, s, &st);
      a.dir[k] = dp;
    }
    if (st != VM_OK) return st;
    a.z = nullptr;
    a.out = pass == 0 ? yr : yc;
    a.batch = batch;
    a.dim = dim;
    a.L = L;
    a.dstate = static_cast<int>(dstate);
    a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
    a.zoh = (options & VM_ZOH) != 0;
    a.reverse = 0;
    a.scale = 1.0f;
    st = launch_bidir(a, /*bf16=*/false, ws, s);
  }
  if (st != VM_OK) return st;
  return hip_status(vmk::launch_ss2d_merge(yr, yc, z, out, batch * dim, height, width,
                                           combine_scale, bf16, s));
}

int vm_ss2d_scan_bwd(const vm_scan_dir *dirs, const void *u, const void *z, const void *dout,
                     float combine_scale, const vm_scan_grad *grads, float *du, void *dz,
                     int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate,
                     int dtype, int options, void *stream) {
  int64_t tok = 0, bc = 0;
  if (!dims_ok({batch, dim, height, width}, &tok)) return VM_ERR_SHAPE;
  const int64_t L = height * width;
  int st = check_bwd_common(dtype, options, batch, dim, L, dstate, z, dout, dz, &tok, &bc);
  if (st != VM_OK) return st;
  if (!std::isfinite(combine_scale) || batch * dim > kMaxPlanes) return VM_ERR_UNSUPPORTED;
  if (((height + 31) / 32) * ((width + 31) / 32) > 65535) return VM_ERR_UNSUPPORTED;
  if (dirs == nullptr || u == nullptr || grads == nullptr || du == nullptr) return VM_ERR_NULL;
  const bool bf16 = dtype == VM_BF16;
  const int es = bf16 ? 2 : 4;
  vm_scan_dir d[4];
  std::vector<Span> ins, outs;
  for (int k = 0; k < 4 && st == VM_OK; ++k) {
    d[k] = dirs[k];
    d[k].u = u;                     // the one map every traversal reads
    st = check_dir(&d[k], tok, tok, batch, L, dim, dstate, es, Span());
    if (st == VM_OK) st = check_bwd_bc(&d[k], L, dstate);
    if (st == VM_OK && d[k].conv_w != nullptr) st = VM_ERR_UNSUPPORTED;
    if (st == VM_OK) dir_spans(&d[k], tok, batch, L, dim, dstate, es, ins);
  }
  if (st != VM_OK) return st;
  ins.push_back(span(z, tok * es));
  ins.push_back(span(dout, tok * es));
  outs.push_back(span(du, tok * 4));
  outs.push_back(span(dz, tok * 4));
  for (const Span &i : ins)
    if (overlaps(outs[0], i) || overlaps(outs[1], i)) return VM_ERR_ALIAS;
  if (overlaps(outs[0], outs[1])) return VM_ERR_ALIAS;
  // each direction's gradients except du (the map's is summed into du)
  for (int k = 0; k < 4 && st == VM_OK; ++k) {
    vm_scan_grad gk = grads[k];
    gk.du = nullptr;
    st = check_grad(&gk, tok, bc, dim, dstate, false, ins, outs, -1, false);
  }
  if (st != VM_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  const int64_t planes = batch * dim;
  // temporary memory first: the transposed map, the recomputed row and
  // column outputs (with z), the output gradient in both layouts, and the
  // four directions' map gradients
  float *ut = ws.get(tok, &st);
  float *yr = z != nullptr ? ws.get(tok, &st) : nullptr;
  float *yc = z != nullptr ? ws.get(tok, &st) : nullptr;
  float *g = ws.get(tok, &st);
  float *gt = ws.get(tok, &st);
  float *dus[4];
  for (int k = 0; k < 4; ++k) dus[k] = ws.get(tok, &st);
  BwdScratch bs[4];
  for (int k = 0; k < 4 && st == VM_OK; ++k) st = bs[k].get(ws, batch, dim, L);
  vmk::ScanArgs a[2] = {};
  for (int pass = 0; pass < 2 && z != nullptr && st == VM_OK; ++pass) {
    a[pass].out = pass == 0 ? yr : yc;
    a[pass].batch = batch;
    a[pass].dim = dim;
    a[pass].L = L;
    a[pass].dstate = static_cast<int>(dstate);
    st = exchange_for(a[pass], false, ws);
  }
  if (st != VM_OK) return st;
  // fp32 views: the map and its transpose; widened delta, B, C with bf16
  const float *u32 = as_f32(u, tok, bf16, ws, s, &st);
  vm_scan_dir w[4];
  for (int k = 0; k < 4 && st == VM_OK; ++k) {
    w[k] = d[k];
    w[k].u = k < 2 ? u32 : ut;
    if (bf16) {
      const int64_t n = bc_extent(batch, dstate, L, d[k].bc_stride);
      w[k].delta = as_f32(d[k].delta, tok, true, ws, s, &st);
      w[k].B = as_f32(d[k].B, n, true, ws, s, &st);
      w[k].C = as_f32(d[k].C, n, true, ws, s, &st);
    }
  }
  if (st == VM_OK) st = hip_status(vmk::launch_transpose(u32, ut, planes, height, width, false, s));
  const float *z32 = as_f32(z, tok, bf16 && z != nullptr, ws, s, &st);
  const float *dout32 = as_f32(dout, tok, bf16, ws, s, &st);
  if (st != VM_OK) return st;
  if (z != nullptr) {
    // the row and column scans' ungated sums, as the forward computes them
    for (int pass = 0; pass < 2 && st == VM_OK; ++pass) {
      a[pass].dir[0] = resolve_dir(&w[2 * pass], batch, dstate, L, false, ws, s, &st);
      a[pass].dir[1] = resolve_dir(&w[2 * pass + 1], batch, dstate, L, false, ws, s, &st);
      a[pass].softplus = (options & VM_DELTA_SOFTPLUS) != 0;
      a[pass].zoh = (options & VM_ZOH) != 0;
      a[pass].scale = 1.0f;
      // the two traversals' checkpoints, for the backward kernels
      a[pass].ck[0] = bs[2 * pass].ck;
      a[pass].ck[1] = bs[2 * pass + 1].ck;
      if (st == VM_OK) st = launch_bidir(a[pass], false, ws, s);
    }
  }
  // the output gradient in both layouts (and dz, from y = y_r + transpose(y_c)):
  // one fused kernel on four-wide tiles, else the transposes and the
  // elementwise gate (the transpose of y_c lands in dus[0], free until the
  // first backward)
  const bool tile4 = vmk::ss2d_tile4_ok(height, width, {yr, yc, z32, dout32, g, gt, dz, du, dus[0], dus[1],
                                                       dus[2], dus[3]});
  if (st == VM_OK && tile4) {
    st = hip_status(vmk::launch_ss2d_gate_bwd(yr, yc, z32, dout32, g, gt, static_cast<float *>(dz), planes,
                                              height, width, combine_scale, s));
  } else if (st == VM_OK) {
    if (z != nullptr) st = hip_status(vmk::launch_transpose(yc, dus[0], planes, width, height, false, s));
    if (st == VM_OK)
      st = hip_status(vmk::launch_gate_bwd(yr, z32, dout32, g, static_cast<float *>(dz), tok, combine_scale,
                                           s, z != nullptr ? dus[0] : nullptr));
    if (st == VM_OK) st = hip_status(vmk::launch_transpose(g, gt, planes, height, width, false, s));
  }
  // the four backward scans in one launch: rows on g, columns on its transpose
  vm_scan_grad gk[4];
  const vm_scan_dir *pk[4];
  const vm_scan_grad *gkp[4];
  const float *dyk[4];
  const int revk[4] = {0, 1, 0, 1};
  for (int k = 0; k < 4; ++k) {
    gk[k] = grads[k];
    gk[k].du = dus[k];
    pk[k] = &w[k];
    gkp[k] = &gk[k];
    dyk[k] = k < 2 ? g : gt;
  }
  if (st == VM_OK)
    st = run_bwd_group(4, pk, dyk, gkp, bs, batch, dim, L, dstate, options, revk, ws, s,
                       z != nullptr ? Prep::kCk : Prep::kNone);
  // du = (du_0 + du_1) + transpose(du_2 + du_3): fused on four-wide tiles,
  // else through g and gt (free now)
  if (st == VM_OK && tile4)
    return hip_status(vmk::launch_ss2d_du_sum(dus[0], dus[1], dus[2], dus[3], du, planes, height, width, s));
  if (st == VM_OK) st = hip_status(vmk::launch_add(dus[2], dus[3], nullptr, g, tok, s));
  if (st == VM_OK) st = hip_status(vmk::launch_transpose(g, gt, planes, width, height, false, s));
  if (st == VM_OK) st = hip_status(vmk::launch_add(dus[0], dus[1], gt, du, tok, s));
  return st;
}

int vm_selective_scan_bwd(const vm_scan_dir *p, const void *z, const void *dout,
                          const vm_scan_grad *g, void *dz, int64_t batch, int64_t dim,
                          int64_t seqlen, int64_t dstate, int dtype, int options, int reverse,
                          void *stream) {
  int64_t tok = 0, bc = 0;
  int st = check_bwd_common(dtype, options, batch, dim, seqlen, dstate, z, dout, dz, &tok, &bc);
  if (st != VM_OK) return st;
  if (!flag_ok(reverse)) return VM_ERR_FLAG;
  const bool bf16 = dtype == VM_BF16;
  const int es = bf16 ? 2 : 4;
  st = check_dir(p, tok, tok, batch, seqlen, dim, dstate, es, Span());
  if (st == VM_OK) st = check_bwd_bc(p, seqlen, dstate);
  if (st != VM_OK) return st;
  const bool conv = p->conv_w != nullptr;
  std::vector<Span> ins, outs;
  dir_spans(p, tok, batch, seqlen, dim, dstate, es, ins);
  ins.push_back(span(z, tok * es));
  ins.push_back(span(dout, tok * es));
  st = check_grad(g, tok, bc, dim, dstate, conv, ins, outs);
  if (st != VM_OK) return st;
  for (const Span &o : outs)
    if (overlaps(span(dz, tok * 4), o)) return VM_ERR_ALIAS;
  for (const Span &i : ins)
    if (overlaps(span(dz, tok * 4), i)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  // temporary memory first, so that a failed allocation launches nothing
  BwdScratch bs;
  st = bs.get(ws, batch, dim, seqlen);
  float *y = z != nullptr ? ws.get(tok, &st) : nullptr;
  float *dyb = z != nullptr ? ws.get(tok, &st) : nullptr;
  ConvBwd cv;
  if (st == VM_OK && conv) st = cv.get(ws, tok, batch, dim);
  if (st != VM_OK) return st;
  // bf16 inputs run the fp32 path on widened copies
  vm_scan_dir w = widen_dir(p, tok, batch, seqlen, dstate, bf16, ws, s, &st);
  const float *z32 = as_f32(z, tok, bf16 && z != nullptr, ws, s, &st);
  const float *dy = as_f32(dout, tok, bf16, ws, s, &st);
  if (st == VM_OK && conv) st = cv.forward(w, batch, dim, seqlen, reverse, s);
  if (st != VM_OK) return st;
  w.conv_w = w.conv_b = nullptr;
  if (z != nullptr) {
    // the ungated forward output, for dz, then dy = dout * SiLU(z)
    vmk::ScanArgs a = {};
    a.dir[0] = a.dir[1] = resolve_dir(&w, batch, dstate, seqlen, false, ws, s, &st);
    a.out = y;
    a.batch = batch;
    a.dim = dim;
    a.L = seqlen;
    a.dstate = static_cast<int>(dstate);
    a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
    a.zoh = (options & VM_ZOH) != 0;
    a.reverse = reverse;
    a.scale = 1.0f;
    const vmk::ScanPlan plan = vmk::plan_scan(batch, dim, seqlen, a.dstate, 1, false);
    if (!vmk::scan_offsets_fit(plan, a, false)) return VM_ERR_UNSUPPORTED;
    st = hip_status(vmk::launch_scan(plan, a, false, s));
    if (st == VM_OK)
      st = hip_status(vmk::launch_gate_bwd(y, z32, dy, dyb, static_cast<float *>(dz), tok, 1.0f, s));
    if (st != VM_OK) return st;
    dy = dyb;
  }
  if (!conv) return run_bwd(&w, dy, g, bs, batch, dim, seqlen, dstate, options, reverse, ws, s);
  vm_scan_grad gu = *g;
  gu.du = cv.du;
  st = run_bwd(&w, dy, &gu, bs, batch, dim, seqlen, dstate, options, reverse, ws, s);
  if (st != VM_OK) return st;
  return cv.backward(*p, g, batch, dim, seqlen, reverse, s);
}

int vm_bidir_scan_bwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd, const void *z,
                      const void *dout, float combine_scale, const vm_scan_grad *gf,
                      const vm_scan_grad *gb, void *dz, int64_t batch, int64_t dim,
                      int64_t seqlen, int64_t dstate, int dtype, int options, void *stream) {
  int64_t tok = 0, bc = 0;
  int st = check_bwd_common(dtype, options, batch, dim, seqlen, dstate, z, dout, dz, &tok, &bc);
  if (st != VM_OK) return st;
  if (!std::isfinite(combine_scale)) return VM_ERR_UNSUPPORTED;
  const bool bf16 = dtype == VM_BF16;
  const int es = bf16 ? 2 : 4;
  st = check_dir(fwd, tok, tok, batch, seqlen, dim, dstate, es, Span());
  if (st == VM_OK) st = check_dir(bwd, tok, tok, batch, seqlen, dim, dstate, es, Span());
  if (st == VM_OK) st = check_bwd_bc(fwd, seqlen, dstate);
  if (st == VM_OK) st = check_bwd_bc(bwd, seqlen, dstate);
  if (st != VM_OK) return st;
  if ((fwd->conv_w == nullptr) != (bwd->conv_w == nullptr)) return VM_ERR_UNSUPPORTED;
  const bool conv = fwd->conv_w != nullptr;
  std::vector<Span> ins, outs;
  dir_spans(fwd, tok, batch, seqlen, dim, dstate, es, ins);
  dir_spans(bwd, tok, batch, seqlen, dim, dstate, es, ins);
  ins.push_back(span(z, tok * es));
  ins.push_back(span(dout, tok * es));
  st = check_grad(gf, tok, bc, dim, dstate, conv, ins, outs);
  if (st == VM_OK) st = check_grad(gb, tok, bc, dim, dstate, conv, ins, outs);
  if (st != VM_OK) return st;
  for (const Span &o : outs)
    if (overlaps(span(dz, tok * 4), o)) return VM_ERR_ALIAS;
  for (const Span &i : ins)
    if (overlaps(span(dz, tok * 4), i)) return VM_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Scratch ws(s);
  // dy = s * dout * SiLU(z) reaches both directions; dz needs y_f + y_b,
  // which the forward kernel recomputes ungated with s = 1.  That
  // recomputation also stores both directions' checkpoints, so that the
  // backward kernels skip their first pass; for short sequences (on-chip
  // exchange) it forms dy and dz itself too.
  const bool fuse = z != nullptr &&
                    vmk::plan_scan(batch, dim, seqlen, static_cast<int>(dstate), 2, false).xmode ==
                        vmk::kXLds;
  float *dy = ws.get(fuse ? vmk::scan_bwd_tiled_floats(batch, dim, seqlen) : tok, &st);
  float *y = z != nullptr && !fuse ? ws.get(tok, &st) : nullptr;
  // per direction: one backward launch for both; with ZOH (launched one
  // direction at a time) the second reuses the first's partial sums
  const bool zoh = (options & VM_ZOH) != 0;
  BwdScratch bs[2];
  st = bs[0].get(ws, batch, dim, seqlen);
  if (st == VM_OK && !zoh) st = bs[1].get(ws, batch, dim, seqlen);
  if (st == VM_OK && zoh) {
    bs[1] = bs[0];
    bs[1].ck = ws.get(vmk::scan_bwd_ck_floats(batch, dim, seqlen), &st);
  }
  ConvBwd cvf, cvb;
  if (st == VM_OK && conv) st = cvf.get(ws, tok, batch, dim);
  if (st == VM_OK && conv) st = cvb.get(ws, tok, batch, dim);
  vmk::ScanArgs a = {};                 // the forward recomputation (with z)
  a.out = fuse ? dy : y;                // (not written when fused)
  a.batch = batch;
  a.dim = dim;
  a.L = seqlen;
  a.dstate = static_cast<int>(dstate);
  if (st == VM_OK && z != nullptr && !fuse) st = exchange_for(a, false, ws);
  if (st != VM_OK) return st;
  // bf16 inputs run the fp32 path on widened copies
  vm_scan_dir wf = widen_dir(fwd, tok, batch, seqlen, dstate, bf16, ws, s, &st);
  vm_scan_dir wb = widen_dir(bwd, tok, batch, seqlen, dstate, bf16, ws, s, &st);
  const float *z32 = as_f32(z, tok, bf16 && z != nullptr, ws, s, &st);
  const float *dout32 = as_f32(dout, tok, bf16, ws, s, &st);
  // with the fused conv each direction scans its own u = SiLU(conv(x)), the
  // backward direction's convolution running in reversed order
  if (st == VM_OK && conv) st = cvf.forward(wf, batch, dim, seqlen, 0, s);
  if (st == VM_OK && conv) st = cvb.forward(wb, batch, dim, seqlen, 1, s);
  if (st != VM_OK) return st;
  wf.conv_w = wf.conv_b = wb.conv_w = wb.conv_b = nullptr;
  if (z != nullptr) {
    a.dir[0] = resolve_dir(&wf, batch, dstate, seqlen, false, ws, s, &st);
    a.dir[1] = resolve_dir(&wb, batch, dstate, seqlen, false, ws, s, &st);
    if (st != VM_OK) return st;
    a.softplus = (options & VM_DELTA_SOFTPLUS) != 0;
    a.zoh = (options & VM_ZOH) != 0;
    a.scale = 1.0f;
    // both directions' checkpoints, so that the backward kernels skip their
    // first pass
    a.ck[0] = bs[0].ck;
    a.ck[1] = bs[1].ck;
    if (fuse) {
      a.gz = z32;
      a.dout = dout32;
      a.dy = dy;
      a.dz = static_cast<float *>(dz);
      a.gscale = combine_scale;
    }
    st = launch_bidir(a, false, ws, s);
    if (st != VM_OK) return st;
  }
  const Prep prep = z == nullptr ? Prep::kNone : fuse ? Prep::kCkDyTiled : Prep::kCk;
  if (!fuse) {
    st = hip_status(vmk::launch_gate_bwd(y, z32, dout32, dy, static_cast<float *>(dz), tok,
                                         combine_scale, s));
    if (st != VM_OK) return st;
  }
  vm_scan_grad guf = *gf, gub = *gb;   // the scans' u gradients (temporary with the conv)
  if (conv) {
    guf.du = cvf.du;
    gub.du = cvb.du;
  }
  if (zoh) {
    st = run_bwd(&wf, dy, &guf, bs[0], batch, dim, seqlen, dstate, options, 0, ws, s, prep);
    if (st == VM_OK) st = run_bwd(&wb, dy, &gub, bs[1], batch, dim, seqlen, dstate, options, 1, ws, s, prep);
  } else {
    const vm_scan_dir *pk[2] = {&wf, &wb};
    const float *dyk[2] = {dy, dy};
    const vm_scan_grad *gk[2] = {&guf, &gub};
    const int revk[2] = {0, 1};
    st = run_bwd_group(2, pk, dyk, gk, bs, batch, dim, seqlen, dstate, options, revk, ws, s, prep);
  }
  if (st == VM_OK && conv) st = cvf.backward(*fwd, gf, batch, dim, seqlen, 0, s);
  if (st == VM_OK && conv) st = cvb.backward(*bwd, gb, batch, dim, seqlen, 1, s);
  return st;
}

}  // extern "C"
