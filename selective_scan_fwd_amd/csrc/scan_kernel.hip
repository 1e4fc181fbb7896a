// Selective scan (S6) forward for gfx950: one direction, or both directions
// of a Vim bidirectional block fused in one workgroup.
//
// Method (Vision Mamba page, "A state retains, writes, and reads" and
// implementation rows 4-5): for each channel d of batch row b, from a zero
// state, dt = softplus(delta + bias), h_n <- exp(dt A_n) h_n + dt B_n u,
// y = sum_n C_n h_n + D u; the backward direction visits t = L-1..0 and the
// two directions are summed, scaled and gated by SiLU(z).
//
// Work decomposition (MI355X-first):
//  * A workgroup owns R consecutive channels of one batch row and runs one
//    wave per direction.  A wave's 64 lanes are (state group, channel): a
//    lane keeps NS = 16 / SPLIT states of one channel in VGPRs and runs the
//    recurrence sequentially in t; R = 64 / SPLIT.  The state split is what
//    yields enough waves to fill 1024 SIMDs on short, narrow problems.
//  * Waves run autonomously.  The only workgroup barrier is at the midpoint
//    of a bidirectional scan (and one before the final write-out).
//  * The sequence is processed in tiles of T steps.  Per tile a wave stages
//    (softplus(delta + bias), u) for its R channels and the tile's B and C
//    values into its LDS, in visit order (a backward tile is stored reversed)
//    so that every lane reads step q at the same immediate offset; softplus is
//    computed once per element.  B and C of a step are held one value per
//    lane of each 16-lane row (the row is one state group) and reach the
//    other lanes as DPP row broadcasts folded into the multiply-adds, so they
//    cost one 4-byte LDS read per lane per step.
//  * Latency is hidden by software pipelining in registers: the global loads
//    of tile k+2 are issued at the start of iteration k.
//  * Bidirectional: phase 1 has the forward wave on the first ceil(nt/2)
//    tiles and the backward wave on the rest; each parks its sums in an
//    exchange buffer.  After the barrier each wave adds its sums to the
//    other's parked values.  For short sequences the exchange block [R][L]
//    sits in LDS and the gated output is written in one flat pass over the
//    workgroup's contiguous [R x L] slab of `out`, so each line is written
//    whole, once.  Long sequences park in fp32 global memory (rows padded to
//    whole cache lines) and finish tile by tile.
#include <type_traits>

#include "vm_internal.h"

namespace vmk {
namespace {

// Broadcast lane J of each 16-lane row (DPP row_newbcast); folds into the
// consuming v_mul_f32 as a DPP operand.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, true));
}

// y += row_bcast<J>(c) * h as one v_fmac_f32_dpp.  c must come straight from
// memory (no VALU write of it just before), which holds for the LDS-loaded
// B/C value it is used with.
template <int J> __device__ __forceinline__ void fmac_row_bcast(float &y, float c, float h);
#define VM_FMAC_BCAST(J)                                                              \
  template <>                                                                         \
  __device__ __forceinline__ void fmac_row_bcast<J>(float &y, float c, float h) {     \
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #J " row_mask:0xf bank_mask:0xf"    \
        : "+v"(y)                                                                     \
        : "v"(c), "v"(h));                                                            \
  }
VM_FMAC_BCAST(4) VM_FMAC_BCAST(5) VM_FMAC_BCAST(6) VM_FMAC_BCAST(7)
VM_FMAC_BCAST(8) VM_FMAC_BCAST(9) VM_FMAC_BCAST(10) VM_FMAC_BCAST(11)
VM_FMAC_BCAST(12) VM_FMAC_BCAST(13) VM_FMAC_BCAST(14) VM_FMAC_BCAST(15)
#undef VM_FMAC_BCAST

template <int NS, int J>
__device__ __forceinline__ void state_step(float (&h)[NS], const float (&A2)[NS], float dt,
                                           float dtu, float bc, float &y) {
  if constexpr (J < NS) {
    const float dA = hw_exp2(dt * A2[J]);
    h[J] = __builtin_fmaf(dA, h[J], dtu * row_bcast<J>(bc));
    fmac_row_bcast<NS + J>(y, bc, h[J]);
    state_step<NS, J + 1>(h, A2, dt, dtu, bc, y);
  }
}

// Workgroup barrier that orders LDS only: global loads issued before it stay
// in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int T, int R>
struct Layout {
  static constexpr int PSTR = 2 * T + 2;                  // (dt, u) per row; PSTR/2 odd
  static constexpr int QSTR = T + 1;                      // partials per lane, odd
  static constexpr int PREP = R * PSTR;
  static constexpr int BC = 32 * T;                       // B in slots 0..15, C in 16..31
  static constexpr int PART = 64 * QSTR;
  static constexpr int WAVE = PREP + BC + PART;           // floats per wave
};

// Row stride of the LDS exchange block: >= L and congruent to T mod 32, so
// that a combine instruction (T consecutive steps of 64/T channels) hits 32
// distinct banks.
__host__ __device__ inline int xchg_stride(int64_t L, int T) {
  return static_cast<int>(L + (((T - L) % 32) + 32) % 32);
}

template <typename Tin, int SPLIT, int DIRS, int XMODE, int T>
__global__ void __launch_bounds__(64 * DIRS)
scan_kernel(const ScanArgs p) {
  constexpr int NS = 16 / SPLIT;                 // states per lane
  constexpr int R = 64 / SPLIT;                  // channels per workgroup
  constexpr int PE = R * T / 64;                 // staged (dt, u) elements per lane per tile
  constexpr int BE = T / 2;                      // staged B/C values per lane per tile
  using Lay = Layout<T, R>;
  static_assert(NS >= 4 && NS <= 8 && R % 16 == 0 && T % 2 == 0 && (R * T) % 64 == 0, "shape");

  extern __shared__ float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float *const prep = smem + wave * Lay::WAVE;   // [R][PSTR]
  float *const bcs = prep + Lay::PREP;           // [T][32]
  float *const part = bcs + Lay::BC;             // [64 lanes][QSTR]
  float *const xlds = smem + DIRS * Lay::WAVE;   // [R][XS]   (kXLds)

  const int sp = lane / R;                       // state group
  const int r = lane % R;                        // channel within the block
  const int dir = wave;                          // 0 forward, 1 backward
  const bool rev = DIRS == 2 ? dir == 1 : p.reverse != 0;

  const int64_t dim = p.dim, L = p.L;
  const int nrb = static_cast<int>((dim + R - 1) / R);
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int b = blk / nrb;
  const int d0 = (blk - b * nrb) * R;
  const int rows = static_cast<int>(dim - d0 < R ? dim - d0 : R);
  const int nt = static_cast<int>((L + T - 1) / T);
  const int XS = xchg_stride(L, T);
  const int dstate = p.dstate;

  const DirPtrs P = p.dir[DIRS == 2 ? wave : 0];  // wave-uniform selection
  const Tin *__restrict__ gu = static_cast<const Tin *>(P.u);
  const Tin *__restrict__ gdl = static_cast<const Tin *>(P.delta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(P.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(P.C);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tin *__restrict__ gout = static_cast<Tin *>(p.out);
  float *__restrict__ gx = p.xglobal;
  const int64_t rowbase = (static_cast<int64_t>(b) * dim + d0) * L;  // element (b, d0, 0)
  const int64_t xbase = (static_cast<int64_t>(b) * dim + d0) * p.xstride;
  const int64_t bcbase = static_cast<int64_t>(b) * P.bsb;

  // ---- scan role: channel d0 + r, states n0 .. n0 + NS - 1 (states at or
  // beyond dstate have A = 0 and zero B/C, so they stay at zero)
  const int n0 = sp * NS;
  const bool lane_ok = r < rows;
  float A2[NS], h[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n0 + j;
    A2[j] = (lane_ok && n < dstate) ? P.A[static_cast<int64_t>(d0 + r) * dstate + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
  }
  const float Dd = (lane_ok && sp == 0) ? P.D[d0 + r] : 0.0f;
  // lane j of each 16-lane row holds B[n0 + j] (j < NS) or C[n0 + j - NS]
  const int rl = lane & 15;
  const int bc_slot = rl < NS ? n0 + rl : (rl < 2 * NS ? 16 + n0 + rl - NS : 0);

  // ---- staging role: element e = lane + 64 i of the R x T tile, (srow, sq)
  // with the visit position sq fastest
  int srow[PE], sq[PE];
  float sbias[PE];
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    const int e = lane + 64 * i;
    srow[i] = e / T;
    sq[i] = e % T;
    sbias[i] = (P.bias != nullptr && srow[i] < rows) ? P.bias[d0 + srow[i]] : 0.0f;
  }

  // Tile of iteration k and the step at visit position q of tile j.
  auto tile_of = [&](int k) __attribute__((always_inline)) { return rev ? nt - 1 - k : k; };
  auto step_of = [&](int j, int q) __attribute__((always_inline)) {
    return static_cast<int64_t>(j) * T + (rev ? T - 1 - q : q);
  };

  // Raw global values of two tiles in flight (index = tile parity).  The loads
  // are unconditional, at clamped in-bounds addresses, and nothing consumes
  // them before the tile is staged: straight-line code with a static count of
  // loads in flight lets the wait for an older tile leave the prefetch just
  // issued in flight.  Which staged elements are real is kept as a bit mask
  // (bit i: element i of the lane lies inside the row block and the sequence).
  float ru[2][PE], rd[2][PE], rbc[2][BE];
  unsigned okm[2];
  const int lastrow = rows - 1;
  bool bc_ok[BE];                                // B/C slot holds a real state
#pragma unroll
  for (int i = 0; i < BE; ++i) bc_ok[i] = ((lane + 64 * i) % 16) < dstate;

  auto stage_load = [&](int k, auto par) __attribute__((always_inline)) {
    constexpr int Q = decltype(par)::value;
    const int j = tile_of(k);
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int64_t t = step_of(j, sq[i]);
      m |= (srow[i] < rows && t < L) ? 1u << i : 0u;
      const int64_t off = rowbase + static_cast<int64_t>(srow[i] < rows ? srow[i] : lastrow) * L +
                          (t < L ? t : L - 1);
      ru[Q][i] = to_f32(gu[off]);
      rd[Q][i] = to_f32(gdl[off]);
    }
    okm[Q] = m;
#pragma unroll
    for (int i = 0; i < BE; ++i) {
      const int e = lane + 64 * i;               // (q, slot) of the T x 32 block
      const int q = e / 32, slot = e % 32, n = slot % 16;
      const int64_t t = step_of(j, q);
      const int64_t off = bcbase + (n < dstate ? n : dstate - 1) * P.bsn + (t < L ? t : L - 1) * P.bst;
      rbc[Q][i] = to_f32((slot < 16 ? gB : gC)[off]);
    }
  };

  // Steps past L and channels past dim stage dt = u = 0, so the state stays
  // where it is (zero before the first real step); B/C slots of states past
  // dstate stage 0.  softplus is evaluated unconditionally and selected, which
  // keeps the loop body free of branches.
  auto stage_store = [&](auto par) __attribute__((always_inline)) {
    constexpr int Q = decltype(par)::value;
    const bool sp_on = p.softplus != 0;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const bool ok = (okm[Q] >> i) & 1u;
      const float x = rd[Q][i] + sbias[i];
      const float sx = softplus_f(x);
      const float dtv = ok ? (sp_on ? sx : x) : 0.0f;
      const float uv = ok ? ru[Q][i] : 0.0f;
      *reinterpret_cast<float2 *>(prep + srow[i] * Lay::PSTR + 2 * sq[i]) = make_float2(dtv, uv);
    }
#pragma unroll
    for (int i = 0; i < BE; ++i) bcs[lane + 64 * i] = bc_ok[i] ? rbc[Q][i] : 0.0f;
  };

  const float *const pr_lane = prep + r * Lay::PSTR;
  const float *const bc_lane = bcs + bc_slot;
  float *const part_lane = part + lane * Lay::QSTR;

  auto do_scan = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const float2 du = *reinterpret_cast<const float2 *>(pr_lane + 2 * q);
      const float bc = bc_lane[q * 32];
      const float dt = du.x, u = du.y;
      const float dtu = dt * u;
      float y = Dd * u;
      state_step<NS, 0>(h, A2, dt, dtu, bc, y);
      part_lane[q] = y;
    }
  };

  // Finishing a tile needs the gate (one direction) or the gate and the
  // parked partials (long bidirectional); they are loaded ahead of the scan.
  float zr[PE], xr[PE];
  auto comb_load = [&](int k, bool second) __attribute__((always_inline)) {
    // (z absent: u stands in as an always-valid address; the value is unused)
    if (XMODE == kXLds || (XMODE == kXGlobal && !second)) return;
    const Tin *const gzl = gz != nullptr ? gz : gu;
    const int j = tile_of(k);
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int64_t t = step_of(j, sq[i]);
      const int64_t tc = t < L ? t : L - 1;
      const int64_t rc = srow[i] < rows ? srow[i] : lastrow;
      zr[i] = to_f32(gzl[rowbase + rc * L + tc]);
      xr[i] = XMODE == kXGlobal ? gx[xbase + rc * p.xstride + tc] : 0.0f;
    }
  };

  auto do_combine = [&](int k, bool second) __attribute__((always_inline)) {
    const int j = tile_of(k);
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int row = srow[i], q = sq[i];
      const int64_t t = step_of(j, q);
      if (row >= rows || t >= L) continue;
      float y = 0.0f;
#pragma unroll
      for (int s = 0; s < SPLIT; ++s) y += part[(s * R + row) * Lay::QSTR + q];
      if (DIRS == 1) {
        const float g = gz != nullptr ? silu_f(zr[i]) : 1.0f;
        gout[rowbase + static_cast<int64_t>(row) * L + t] = from_f32<Tin>(y * g);
      } else if (XMODE == kXLds) {
        float *xp = xlds + row * XS + t;
        *xp = second ? *xp + y : y;
      } else if (!second) {
        gx[xbase + static_cast<int64_t>(row) * p.xstride + t] = y;
      } else {
        const float g = gz != nullptr ? silu_f(zr[i]) : 1.0f;
        gout[rowbase + static_cast<int64_t>(row) * L + t] = from_f32<Tin>(p.scale * (y + xr[i]) * g);
      }
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // Tiles of phase 1: forward ceil(nt/2), backward the rest (first visits).
  const int half = (nt + 1) / 2;
  const int n1 = DIRS == 1 ? nt : (dir == 0 ? half : nt - half);

  // One iteration k (register parity Q): issue the finishing loads of k and
  // the loads of tile k+2, scan k, stage k+1, combine k.  A wave's LDS
  // traffic executes in program order, so none of this needs a barrier.  The
  // prefetch and the staging run on every iteration (past the end they repeat
  // the last tile, whose staged copy is never scanned): a load issued under a
  // branch would make the count of loads in flight path-dependent, and the
  // wait before staging would then also wait for the prefetch.
  auto iteration = [&](int k, auto par) __attribute__((always_inline)) {
    constexpr int Q = decltype(par)::value;
    using Qn = std::integral_constant<int, 1 - Q>;
    const bool second = k >= n1;
    if (DIRS == 2 && k == n1) {
      // midpoint: every first visit of both waves is parked
      if (XMODE == kXGlobal) __syncthreads();
      else lds_barrier();
    }
    comb_load(k, second);
    stage_load(k + 2 < nt ? k + 2 : nt - 1, par);
    do_scan();
    stage_store(Qn());
    do_combine(k, second);
  };

  stage_load(0, P0());
  stage_load(nt > 1 ? 1 : 0, P1());
  stage_store(P0());
  int k = 0;
  for (; k + 1 < nt; k += 2) {
    iteration(k, P0());
    iteration(k + 1, P1());
  }
  if (k < nt) iteration(k, P0());
  if (DIRS == 2 && n1 == nt) {                 // a wave with no second-phase tiles
    if (XMODE == kXGlobal) __syncthreads();
    else lds_barrier();
  }

  // ---- short bidirectional sequences: gate and write the workgroup's whole
  // [rows x L] slab of out in flat order (coalesced, whole lines).
  if (DIRS == 2 && XMODE == kXLds) {
    lds_barrier();
    const int64_t n = static_cast<int64_t>(rows) * L;
    const int tid = threadIdx.x;
    int fr = tid / static_cast<int>(L), ft = tid % static_cast<int>(L);
    for (int64_t f = tid; f < n; f += 64 * DIRS) {
      float y = p.scale * xlds[fr * XS + ft];
      if (gz != nullptr) y *= silu_f(to_f32(gz[rowbase + f]));
      gout[rowbase + f] = from_f32<Tin>(y);
      ft += 64 * DIRS;
      while (ft >= L) { ft -= static_cast<int>(L); ++fr; }
    }
  }
}

template <typename Tin, int SPLIT, int DIRS, int XMODE, int T>
hipError_t launch_one(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  auto kern = scan_kernel<Tin, SPLIT, DIRS, XMODE, T>;
  static bool attr_set = false;  // benign race: the attribute value is idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(plan.blocks)), dim3(plan.threads), plan.lds,
                     s, a);
  return hipGetLastError();
}

template <typename Tin, int SPLIT>
hipError_t dispatch_mode(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (plan.dirs == 1) return launch_one<Tin, SPLIT, 1, kXNone, 16>(plan, a, s);
  if (plan.xmode == kXLds) return launch_one<Tin, SPLIT, 2, kXLds, 8>(plan, a, s);
  return launch_one<Tin, SPLIT, 2, kXGlobal, 8>(plan, a, s);
}

template <typename Tin>
hipError_t dispatch_dtype(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (plan.S == 2) return dispatch_mode<Tin, 2>(plan, a, s);
  return dispatch_mode<Tin, 4>(plan, a, s);
}

size_t lds_bytes(int split, int dirs, int T, int xmode, int64_t L) {
  const int R = 64 / split;
  size_t f = static_cast<size_t>(dirs) * (R * (2 * T + 2) + 32 * T + 64 * (T + 1));
  if (xmode == kXLds) f += static_cast<size_t>(R) * xchg_stride(L, T);
  return f * sizeof(float);
}

}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t L, int dstate, int dirs) {
  (void)dstate;
  ScanPlan pl{};
  pl.dirs = dirs;
  pl.threads = 64 * dirs;
  // Split each channel's 16 states over 2 lanes, or over 4 when that leaves
  // fewer than two waves per SIMD.
  auto waves = [&](int split) { return batch * ((dim * split + 63) / 64) * dirs; };
  pl.S = waves(2) >= 2048 ? 2 : 4;
  pl.blocks = batch * ((dim + 64 / pl.S - 1) / (64 / pl.S));
  if (dirs == 1) {
    pl.T = 16;
    pl.xmode = kXNone;
  } else {
    // On-chip exchange while four workgroups still fit a CU's 160 KB LDS.
    pl.T = 8;
    pl.xmode = lds_bytes(pl.S, 2, 8, kXLds, L) <= 40 * 1024 ? kXLds : kXGlobal;
  }
  pl.lds = lds_bytes(pl.S, dirs, pl.T, pl.xmode, L);
  return pl;
}

int64_t xchg_global_stride(int64_t L) { return (L + 31) / 32 * 32; }

hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &args, bool bf16, hipStream_t s) {
  if (plan.blocks <= 0) return hipSuccess;
  return bf16 ? dispatch_dtype<bf16_t>(plan, args, s) : dispatch_dtype<float>(plan, args, s);
}

}  // namespace vmk
