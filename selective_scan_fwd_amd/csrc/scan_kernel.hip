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
//  * A workgroup owns 64 consecutive channels of one batch row.  Each wave's
//    64 lanes are those 64 channels; every lane keeps its channel's state in
//    VGPRs and runs the recurrence sequentially in t.
//  * The 16 states of a direction are split over S waves (NS = 16/S states
//    each).  Within a wave, B and C are therefore wave-uniform and are read
//    with scalar loads into SGPRs: no LDS or vector traffic for them.  The
//    split multiplies the wave count by S, which is what fills 1024 SIMDs on
//    short, narrow problems.
//  * The sequence is processed in tiles of T steps.  Per tile the S waves of
//    a direction cooperatively stage (dt, u) into LDS with coalesced loads
//    (softplus is computed once per element, not once per wave), scan, and
//    leave per-wave partial outputs in LDS; after one barrier the partials are
//    summed and written with coalesced stores.
//  * Bidirectional: the forward waves walk tiles 0..nt-1 while the backward
//    waves walk nt-1..0 in the same workgroup.  The first direction to reach
//    a tile parks its sum in an exchange buffer (LDS for short sequences,
//    fp32 global memory otherwise); the second adds its own, applies
//    scale * SiLU(z) and writes the output, so out is written exactly once.
#include <type_traits>

#include "vm_internal.h"

namespace vmk {
namespace {

typedef __attribute__((address_space(4))) const float *smem_ptr_t;  // scalar-load view

// Uniform (wave-wide) load through the scalar data cache.
__device__ __forceinline__ float sload(const float *p) { return *(smem_ptr_t)p; }

template <int T, int S, int DIRS>
struct Layout {
  static constexpr int PSTR = 2 * T + 2;                 // (dt, u) pairs per row, padded
  static constexpr int QSTR = T + 1;                     // partial outputs per row, padded
  static constexpr int PREP = DIRS * kRows * PSTR;       // floats per prep buffer
  static constexpr int PART = DIRS * S * kRows * QSTR;   // floats per partial buffer
  static constexpr size_t fixed_bytes() { return sizeof(float) * 2 * (PREP + PART); }
};

template <typename Tin, int NS, int S, int DIRS, int XMODE, int T, int TB>
__global__ void __launch_bounds__(kRows * S * DIRS)
scan_kernel(const ScanArgs p) {
  using Lay = Layout<T, S, DIRS>;
  constexpr int NTHR = kRows * S * DIRS;
  constexpr int PE = T / S;                     // prep elements per lane per tile
  static_assert(T % S == 0 && T % TB == 0, "tile shape");
  static_assert(NS * S == 16, "16 state slots per direction");

  extern __shared__ float smem[];
  float *const prep = smem;                      // [2][DIRS][kRows][PSTR]
  float *const part = smem + 2 * Lay::PREP;      // [2][DIRS][S][kRows][QSTR]
  float *const xlds = part + 2 * Lay::PART;      // [kRows][XS]  (kXLds)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int dir = wave / S;
  const int sg = wave - dir * S;

  const int64_t dim = p.dim, L = p.L;
  const int nrb = static_cast<int>((dim + kRows - 1) / kRows);
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int b = blk / nrb;
  const int d0 = (blk - b * nrb) * kRows;
  const int rows = static_cast<int>(dim - d0 < kRows ? dim - d0 : kRows);
  const int nt = static_cast<int>((L + T - 1) / T);
  const int XS = static_cast<int>(L | 1);
  const int dstate = p.dstate;
  const bool rev = (DIRS == 2) ? (dir == 1) : (p.reverse != 0);

  const DirPtrs P = p.dir[dir];
  const Tin *__restrict__ gu = static_cast<const Tin *>(P.u);
  const Tin *__restrict__ gdl = static_cast<const Tin *>(P.delta);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tin *__restrict__ gout = static_cast<Tin *>(p.out);
  float *__restrict__ gx = p.xglobal;
  const int64_t rowbase = (static_cast<int64_t>(b) * dim + d0) * L;  // element (b, d0, 0)
  const int n0 = sg * NS;
  // This wave's B values at bcw[t * 32 + j], C values at bcw[t * 32 + 16 + j].
  const float *__restrict__ bcw = P.BC + static_cast<int64_t>(b) * L * kBCStride + n0;

  // ---- scan role: lane = channel d0 + lane, states n0 .. n0 + NS - 1.  States
  // at or beyond dstate have A = 0 and zero B/C, so they stay at zero.
  const bool lane_ok = lane < rows;
  float A2[NS], h[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n0 + j;
    const bool ok = lane_ok && n < dstate;
    A2[j] = ok ? P.A[static_cast<int64_t>(d0 + lane) * dstate + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
  }
  const float Dd = (lane_ok && sg == 0) ? P.D[d0 + lane] : 0.0f;

  // ---- prep role: element e = sg*64 + lane + i*S*64 of the 64 x T tile
  int prow[PE], ptt[PE];
  float pbias[PE];
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    const int e = sg * kRows + lane + i * S * kRows;
    prow[i] = e / T;
    ptt[i] = e % T;
    pbias[i] = (P.bias != nullptr && prow[i] < rows) ? P.bias[d0 + prow[i]] : 0.0f;
  }

  auto tile_of = [&](int k) { return rev ? nt - 1 - k : k; };

  auto do_prep = [&](int k, int buf) {
    const int j = tile_of(k);
    float *pb = prep + buf * Lay::PREP + dir * kRows * Lay::PSTR;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int row = prow[i], tt = ptt[i];
      const int64_t t = static_cast<int64_t>(j) * T + tt;
      float dtv = 0.0f, uv = 0.0f;
      if (row < rows && t < L) {
        const int64_t off = rowbase + static_cast<int64_t>(row) * L + t;
        uv = to_f32(gu[off]);
        const float x = to_f32(gdl[off]) + pbias[i];
        dtv = p.softplus ? softplus_f(x) : x;
      }
      *reinterpret_cast<float2 *>(pb + row * Lay::PSTR + 2 * tt) = make_float2(dtv, uv);
    }
  };

  auto do_scan = [&](int k, int buf, auto rev_tag) {
    constexpr bool REV = decltype(rev_tag)::value;
    const int j = REV ? nt - 1 - k : k;
    const float *pr = prep + buf * Lay::PREP + dir * kRows * Lay::PSTR + lane * Lay::PSTR;
    float *q = part + buf * Lay::PART + (dir * S + sg) * kRows * Lay::QSTR + lane * Lay::QSTR;
    const int64_t t0 = static_cast<int64_t>(j) * T;
#pragma unroll
    for (int bi = 0; bi < T / TB; ++bi) {
      const int bb = REV ? T / TB - 1 - bi : bi;
      const int64_t tb0 = t0 + bb * TB;
      const bool full = tb0 + TB <= L;
      float Bs[NS][TB], Cs[NS][TB];
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        // Ragged tail: steps past L read the last record; their dt = u = 0.
        int64_t t = tb0 + i;
        if (!full) t = t < L ? t : L - 1;
        const float *ri = bcw + t * kBCStride;
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) {
          Bs[jj][i] = sload(ri + jj);
          Cs[jj][i] = sload(ri + 16 + jj);
        }
      }
#pragma unroll
      for (int ii = 0; ii < TB; ++ii) {
        const int i = REV ? TB - 1 - ii : ii;
        const int tt = bb * TB + i;
        const float2 du = *reinterpret_cast<const float2 *>(pr + 2 * tt);
        const float dt = du.x, u = du.y;
        const float dtu = dt * u;
        float y = Dd * u;
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) {
          const float dA = hw_exp2(dt * A2[jj]);
          h[jj] = __builtin_fmaf(dA, h[jj], dtu * Bs[jj][i]);
          y = __builtin_fmaf(Cs[jj][i], h[jj], y);
        }
        q[tt] = y;
      }
    }
  };

  // Sum of the partial outputs of one tile for direction set [dlo, dhi].
  auto tile_sum = [&](int buf, int dlo, int dhi, int row, int tt) {
    float y = 0.0f;
    for (int dd = dlo; dd <= dhi; ++dd)
#pragma unroll
      for (int s = 0; s < S; ++s)
        y += part[buf * Lay::PART + ((dd * S + s) * kRows + row) * Lay::QSTR + tt];
    return y;
  };

  auto gate = [&](int64_t off) { return gz != nullptr ? silu_f(to_f32(gz[off])) : 1.0f; };

  // Combine one tile: elements first .. 64*T-1 with the given stride.
  // mode 0: one-direction output; 1: first visit (park); 2: second visit
  // (add parked, finish); 3: both directions in this tile (finish).
  auto do_combine = [&](int j, int buf, int mode, int dlo, int dhi, int first, int stride) {
    for (int e = first; e < kRows * T; e += stride) {
      const int row = e / T, tt = e % T;
      const int64_t t = static_cast<int64_t>(j) * T + tt;
      if (row >= rows || t >= L) continue;
      float y = tile_sum(buf, dlo, dhi, row, tt);
      const int64_t off = rowbase + static_cast<int64_t>(row) * L + t;
      if (mode == 0) {
        gout[off] = from_f32<Tin>(y * gate(off));
      } else if (mode == 1) {
        if (XMODE == kXLds) xlds[row * XS + t] = y;
        else gx[off] = y;
      } else {
        if (mode == 2) y += (XMODE == kXLds) ? xlds[row * XS + t] : gx[off];
        gout[off] = from_f32<Tin>(p.scale * y * gate(off));
      }
    }
  };

  // ---- main loop: scan(k) ; prep(k+1) ; barrier ; combine(k)
  do_prep(0, 0);
  __syncthreads();
  for (int k = 0; k < nt; ++k) {
    const int buf = k & 1;
    if (rev) do_scan(k, buf, std::integral_constant<bool, true>());
    else do_scan(k, buf, std::integral_constant<bool, false>());
    if (k + 1 < nt) do_prep(k + 1, buf ^ 1);
    __syncthreads();
    if (DIRS == 1) {
      do_combine(tile_of(k), buf, 0, 0, 0, sg * kRows + lane, S * kRows);
    } else if (2 * k == nt - 1) {
      do_combine(k, buf, 3, 0, 1, tid, NTHR);
    } else {
      const int mode = (2 * k < nt - 1) ? 1 : 2;
      do_combine(tile_of(k), buf, mode, dir, dir, sg * kRows + lane, S * kRows);
    }
  }
}

template <typename Tin, int S, int DIRS, int XMODE, int T>
hipError_t launch_one(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  constexpr int NS = 16 / S;
  constexpr int TB = (16 / NS) < T ? (16 / NS) : T;   // 2*NS*TB <= 32 SGPRs per B/C block
  auto kern = scan_kernel<Tin, NS, S, DIRS, XMODE, T, TB>;
  static bool attr_set = false;  // benign race: the attribute value is idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(plan.blocks)), dim3(plan.threads),
                     plan.lds, s, a);
  return hipGetLastError();
}

template <typename Tin, int S>
hipError_t dispatch_mode(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (plan.dirs == 1) return launch_one<Tin, S, 1, kXNone, 8>(plan, a, s);
  if (plan.xmode == kXLds) {
    if (plan.T == 4) return launch_one<Tin, S, 2, kXLds, 4>(plan, a, s);
    return launch_one<Tin, S, 2, kXLds, 8>(plan, a, s);
  }
  return launch_one<Tin, S, 2, kXGlobal, 8>(plan, a, s);
}

template <typename Tin>
hipError_t dispatch_dtype(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (plan.S == 2) return dispatch_mode<Tin, 2>(plan, a, s);
  return dispatch_mode<Tin, 4>(plan, a, s);
}

size_t fixed_lds(int S, int T, int dirs) {
  const size_t pstr = 2 * T + 2, qstr = T + 1;
  return sizeof(float) * 2 * (dirs * kRows * pstr + dirs * S * kRows * qstr);
}

}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t L, int dstate, int dirs) {
  (void)dstate;
  ScanPlan pl{};
  const int64_t nrb = (dim + kRows - 1) / kRows;
  pl.blocks = batch * nrb;
  pl.dirs = dirs;
  // Fill the 1024 SIMDs: split the 16 states over more waves when row blocks
  // are scarce.
  pl.S = (pl.blocks * dirs * 2 >= 2048) ? 2 : 4;
  pl.threads = kRows * pl.S * dirs;
  // Keep at least two workgroups per CU (160 KB LDS) where possible.
  const size_t kTwoPerCu = 80 * 1024;
  if (dirs == 1) {
    pl.T = 8;
    pl.xmode = kXNone;
    pl.lds = fixed_lds(pl.S, pl.T, 1);
    return pl;
  }
  const size_t x = sizeof(float) * kRows * static_cast<size_t>(L | 1);
  if (fixed_lds(pl.S, 8, 2) + x <= kTwoPerCu) {
    pl.T = 8;
    pl.xmode = kXLds;
    pl.lds = fixed_lds(pl.S, 8, 2) + x;
  } else if (fixed_lds(pl.S, 4, 2) + x <= kTwoPerCu) {
    pl.T = 4;
    pl.xmode = kXLds;
    pl.lds = fixed_lds(pl.S, 4, 2) + x;
  } else {
    pl.T = 8;
    pl.xmode = kXGlobal;
    pl.lds = fixed_lds(pl.S, 8, 2);
  }
  return pl;
}

hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &args, bool bf16, hipStream_t s) {
  if (plan.blocks <= 0) return hipSuccess;
  return bf16 ? dispatch_dtype<bf16_t>(plan, args, s) : dispatch_dtype<float>(plan, args, s);
}

}  // namespace vmk
