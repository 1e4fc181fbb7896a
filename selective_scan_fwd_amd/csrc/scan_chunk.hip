// Sequence-parallel (chunked) selective scan, one direction, for problems
// with too few rows to fill the chip (the single-direction Vim scan of one
// image: 384 channels).
//
// Method (Vision Mamba page, "A state retains, writes, and reads"): per
// channel, from a zero state, h_t = a_t h_{t-1} + w_t with a_t = exp(dt_t A)
// and w_t = dt_t B_t u_t (or the zero-order-hold write), y_t = C_t h_t +
// D u_t, gated by SiLU(z).  The recurrence is affine in h, so a run of steps
// acts on its entry state as h -> P h + g, with P the product of its a_t
// (= 2^(A log2e * its sum of dt)) and g its end state from a zero entry, and
// two runs compose as (P2, g2) o (P1, g1) = (P2 P1, P2 g1 + g2).  The FastVim
// summary ("Technical Contribution", "Core Problem") names the parallel depth
// over the sequence as the cost of scanning long flattened images; this
// kernel spends it where the rows alone leave the chip idle.
//
// Work decomposition:
//  * One workgroup per channel (b, d): four waves, one per group of four
//    states.  Lane l of every wave owns the sub-chunk of visit positions
//    [l Ls, (l + 1) Ls) of the channel's sequence: the 64 lanes cover it.
//  * Pass 1: each lane runs its sub-chunk from a zero state, keeping only
//    the state (g) and the sum of its dt (P = 2^(A log2e sum)).
//  * The 64 (P, g) pairs of a wave are combined in lane order by a
//    Kogge-Stone scan (lane shuffles at distances 1, 2, .., 32); lane l's
//    entry state is the combined state of lanes 0 .. l-1.
//  * The channel's row is staged in LDS first by all 256 threads with
//    coalesced loads: (dt, dt u, u) per step (softplus and the conv computed
//    once per step) and B, C per step as four float4 groups of states, laid
//    out so that the lanes' strided reads hit distinct banks.  Sequences of
//    at most 256 steps (4 per lane) fit.
//  * Pass 2: each lane reruns its sub-chunk from that entry state with the
//    readout; the four waves' partial readouts meet in LDS and are finished
//    (sum, D u, gate) by all threads in step order, coalesced.
//  * The arithmetic is about twice the sequential scan's (the state pass is
//    repeated), which the otherwise idle SIMDs absorb; the critical path is
//    two sub-chunks plus six shuffle rounds instead of the sequence.
//  Global accesses go through buffer resources: positions past the sequence
//  and states past dstate read 0 and drop stores.
#include <type_traits>

#include "scan_device.h"
#include "vm_internal.h"

namespace vmk {
namespace {

constexpr int kLNS = 4;        // states per lane (one wave per group of four)
constexpr int kLMax = 256;     // longest sequence staged (4 steps per lane)
// Staged float4 records (per-step values, and B, C per state group) are
// stored at index i + i / 16: lanes reading every Ls-th record (Ls <= 4)
// then hit 16 distinct bank groups.
__device__ __forceinline__ int skew(int i) { return i + (i >> 4); }
constexpr int kLRec = kLMax + kLMax / 16;  // records per staged array

template <typename Tin, int OPT>
__global__ void __launch_bounds__(256) scan_lane_kernel(const ScanArgs p, int Ls) {
  constexpr bool ZOH = (OPT & kOptZoh) != 0;
  constexpr bool CONV = (OPT & kOptConv) != 0;
  constexpr uint32_t ES = sizeof(Tin);
  // [step] (dt, write factor, u, -); [state group][step] B and C; the partial
  // readouts [state group][step] (the conv input row shares their area)
  __shared__ float4 sE[kLRec];
  __shared__ float4 sB[4][kLRec];
  __shared__ float4 sC[4][kLRec];
  __shared__ float sY[4][kLMax];
  const int tid = threadIdx.x;
  const int sp = __builtin_amdgcn_readfirstlane(tid >> 6);   // state group
  const int lane = tid & 63;
  const int n0 = sp * kLNS;
  const int64_t dim = p.dim;
  const int L = static_cast<int>(p.L);
  const int row = blockIdx.x;                         // b * dim + d
  const int b = static_cast<int>(row / dim);
  const int d = static_cast<int>(row - static_cast<int64_t>(b) * dim);
  const int dstate = p.dstate;
  const bool rev = p.reverse != 0;
  const bool gated = p.z != nullptr;
  const bool sp_on = p.softplus != 0;
  const DirPtrs P = p.dir[0];

  const int64_t rowbase = static_cast<int64_t>(row) * L;
  const uint32_t rowbytes = static_cast<uint32_t>(L) * ES;
  const Rsrc rU = make_rsrc(static_cast<const Tin *>(P.u) + rowbase, rowbytes);
  const Rsrc rD = make_rsrc(static_cast<const Tin *>(P.delta) + rowbase, rowbytes);
  const Rsrc rZ = make_rsrc(gated ? static_cast<const Tin *>(p.z) + rowbase : nullptr, gated ? rowbytes : 0u);
  const Rsrc rO = make_rsrc(static_cast<Tin *>(p.out) + rowbase, rowbytes);
  const uint32_t bcext = (static_cast<uint32_t>(dstate - 1) * static_cast<uint32_t>(P.bsn) +
                          static_cast<uint32_t>(L - 1) * static_cast<uint32_t>(P.bst) + 1) * ES;
  const Rsrc rB = make_rsrc(static_cast<const Tin *>(P.B) + static_cast<int64_t>(b) * P.bsb, bcext);
  const Rsrc rC = make_rsrc(static_cast<const Tin *>(P.C) + static_cast<int64_t>(b) * P.bsb, bcext);

  // ---- stage the row.  Thread tid takes steps t = tid (L <= 256) for the
  // per-step values, and for B and C the (step, state) pairs e = tid + 256 k
  // with the state fastest (consecutive in token-major memory).
  const float bias = P.bias != nullptr ? P.bias[d] : 0.0f;
  const float Dd = P.D[d];
  const int t = tid;                                   // original step of this thread
  const bool tin = t < L;
  const uint32_t to = pin_u(tin ? static_cast<uint32_t>(t) * ES : kOob);
  float x = bload<Tin>(rU, to);
  const float dl = bload<Tin>(rD, to) + bias;
  float bv[16], cv[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = tid + 256 * k;
    const int te = e >> 4, n = e & 15;
    const uint32_t o = pin_u(te < L && n < dstate ? (static_cast<uint32_t>(n) * static_cast<uint32_t>(P.bsn) +
                                                     static_cast<uint32_t>(te) * static_cast<uint32_t>(P.bst)) * ES
                                                  : kOob);
    bv[k] = bload<Tin>(rB, o);
    cv[k] = bload<Tin>(rC, o);
  }
  // the step's position in visit order, and its record
  const int sv = rev ? L - 1 - t : t;
  float u = x;
  if constexpr (CONV) {
    // u = SiLU(b + w0 x[-3] + w1 x[-2] + w2 x[-1] + w3 x[0]) in visit order:
    // the row's inputs meet in LDS (in the partial-readout area)
    float *const sx = &sY[0][0];
    if (tin) sx[sv] = x;
    __syncthreads();
    float v = P.cb != nullptr ? P.cb[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = sv - 3 + k;
      v = __builtin_fmaf(P.cw[static_cast<int64_t>(d) * 4 + k], s >= 0 && tin ? sx[s] : 0.0f, v);
    }
    u = silu_f(v);
    __syncthreads();
  }
  const float dtv = sp_on ? softplus_f(dl) : dl;
  if (tin) sE[skew(sv)] = make_float4(dtv, ZOH ? u : dtv * u, u, 0.0f);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = tid + 256 * k;
    const int te = e >> 4, n = e & 15;
    if (te < L) {
      const int se = skew(rev ? L - 1 - te : te);
      reinterpret_cast<float *>(&sB[n >> 2][se])[n & 3] = bv[k];
      reinterpret_cast<float *>(&sC[n >> 2][se])[n & 3] = cv[k];
    }
  }

  // parameters of channel d (states past dstate: A = 0, B = C = 0, so they stay zero)
  float A2[kLNS], iA[kLNS], h[kLNS];
#pragma unroll
  for (int j = 0; j < kLNS; ++j) {
    const int n = n0 + j;
    const float a = n < dstate ? P.A[static_cast<int64_t>(d) * dstate + n] : 0.0f;
    iA[j] = ZOH && a != 0.0f ? 1.0f / a : 0.0f;
    A2[j] = a * kLog2e;
    h[j] = 0.0f;
  }
  __syncthreads();

  const int s_lo = lane * Ls;                         // this lane's visit range
  const int s_hi = s_lo + Ls < L ? s_lo + Ls : L;
  // one step at visit position s; returns the partial readout (READ)
  auto step = [&](int s, auto read) __attribute__((always_inline)) {
    constexpr bool READ = decltype(read)::value;
    const float4 e = sE[skew(s)];
    const float4 bq = sB[sp][skew(s)];
    const float bj[4] = {bq.x, bq.y, bq.z, bq.w};
    float cj[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (READ) {
      const float4 cq = sC[sp][skew(s)];
      cj[0] = cq.x;
      cj[1] = cq.y;
      cj[2] = cq.z;
      cj[3] = cq.w;
    }
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < kLNS; ++j) {
      const float x2 = e.x * A2[j];
      const float dA = hw_exp2(x2);
      float w = e.y * bj[j];
      if constexpr (ZOH) w *= zoh_coef(e.x, x2, dA, iA[j]);
      h[j] = __builtin_fmaf(dA, h[j], w);
      if constexpr (READ) y = __builtin_fmaf(cj[j], h[j], y);
    }
    return y;
  };

  // ---- pass 1: the sub-chunk's end state from zero and its sum of dt
  float S = 0.0f;
  for (int s = s_lo; s < s_hi; ++s) {
    step(s, std::false_type());
    S += sE[skew(s)].x;
  }

  // ---- lane scan of (P, g): after it, lane l holds the combination of
  // lanes 0 .. l (identity (1, 0) for an empty sub-chunk)
  float Pj[kLNS];
#pragma unroll
  for (int j = 0; j < kLNS; ++j) Pj[j] = hw_exp2(A2[j] * S);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < kLNS; ++j) {
      const float Pl = __shfl_up(Pj[j], off, 64);
      const float gl = __shfl_up(h[j], off, 64);
      if (lane >= off) {
        h[j] = __builtin_fmaf(Pj[j], gl, h[j]);
        Pj[j] *= Pl;
      }
    }
  }
  // entry state of lane l: the combination of lanes 0 .. l-1 applied to 0
#pragma unroll
  for (int j = 0; j < kLNS; ++j) {
    const float gl = __shfl_up(h[j], 1, 64);
    h[j] = lane >= 1 ? gl : 0.0f;
  }

  // ---- pass 2: readout from the entry state; partial readouts by step
  for (int s = s_lo; s < s_hi; ++s) sY[sp][s] = step(s, std::true_type());
  __syncthreads();
  // finishing, thread tid on original step t: sum, D u, gate, store
  if (tin) {
    float y = (sY[0][sv] + sY[1][sv]) + (sY[2][sv] + sY[3][sv]);
    y = __builtin_fmaf(Dd, u, y);
    if (gated) y *= silu_f(bload<Tin>(rZ, to));
    bstore<Tin>(rO, to, y);
  }
}

template <typename Tin, int OPT>
hipError_t launch_lane(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((scan_lane_kernel<Tin, OPT>), dim3(static_cast<unsigned>(plan.blocks)), dim3(256), 0, s,
                     a, plan.chunk_len);
  return hipGetLastError();
}

template <typename Tin>
hipError_t dispatch_lane(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  switch ((a.zoh ? kOptZoh : 0) | (a.conv ? kOptConv : 0)) {
    case 0: return launch_lane<Tin, 0>(plan, a, s);
    case kOptZoh: return launch_lane<Tin, kOptZoh>(plan, a, s);
    case kOptConv: return launch_lane<Tin, kOptConv>(plan, a, s);
    default: return launch_lane<Tin, kOptZoh | kOptConv>(plan, a, s);
  }
}

}  // namespace

hipError_t launch_scan_chunked(const ScanPlan &plan, const ScanArgs &a, bool bf16, hipStream_t s) {
  if (plan.blocks <= 0) return hipSuccess;
  return bf16 ? dispatch_lane<bf16_t>(plan, a, s) : dispatch_lane<float>(plan, a, s);
}

}  // namespace vmk
