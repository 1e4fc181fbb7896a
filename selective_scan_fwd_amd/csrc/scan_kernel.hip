// Selective scan (S6) forward for gfx950: one direction, or both directions
// of a Vim bidirectional block fused in one workgroup.
//
// Method (Vision Mamba page, "A state retains, writes, and reads" and
// implementation rows 4-5): for each channel d of batch row b, from a zero
// state, dt = softplus(delta + bias), h_n <- exp(dt A_n) h_n + dt B_n u,
// y = sum_n C_n h_n + D u; the backward direction visits t = L-1..0 and the
// two directions are summed, scaled and gated by SiLU(z).  Optionally the
// write uses the zero-order-hold coefficient (exp(dt A_n) - 1) / A_n in place
// of dt ("Norm or Direction?" page, section 3, eq. 2), and optionally the
// scan input is computed in the staging pass as u = SiLU(conv(x)), the
// depthwise width-4 causal convolution of the released Vim block ("Inside the
// released Vim block"), causal in each direction's own visit order.
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
//    cost one 4-byte LDS read per lane per step.  Long bidirectional
//    sequences with few rows split a channel's states over 8 lanes instead
//    (two per lane, eight channels per wave, twice the waves); a 16-lane row
//    then holds two state groups, and each lane reads its own B and C pair
//    as one 16-byte LDS value per step.
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
#include <climits>
#include <type_traits>
#include <utility>

#include "scan_device.h"
#include "vm_internal.h"

namespace vmk {
namespace {

// One step of the lane's NS states: h_j <- 2^(dt A2_j) h_j + dtu B_j and
// y = sum_j C_j h_j (B_j, C_j broadcast from lanes j and NS + j of the row).
template <int NS, int J>
__device__ __forceinline__ void state_step(float (&h)[NS], const float (&A2)[NS], float dt,
                                           float dtu, float bc, float &y) {
  if constexpr (J < NS) {
    const float dA = hw_exp2(dt * A2[J]);
    h[J] = __builtin_fmaf(dA, h[J], dtu * row_bcast<J>(bc));
    if constexpr (J == 0) y = row_bcast<NS>(bc) * h[0];
    else fmac_row_bcast<NS + J>(y, bc, h[J]);
    state_step<NS, J + 1>(h, A2, dt, dtu, bc, y);
  }
}

// The same step with the zero-order-hold write k_j u B_j, k_j = expm1(x) / A_j
// for x = dt A_j (here u arrives in place of dt u; zoh_coef has the
// coefficient and its accuracy).
template <int NS, int J>
__device__ __forceinline__ void state_step_zoh(float (&h)[NS], const float (&A2)[NS],
                                               const float (&iA)[NS], float dt, float u,
                                               float bc, float &y) {
  if constexpr (J < NS) {
    const float x2 = dt * A2[J];
    const float dA = hw_exp2(x2);
    const float k = zoh_coef(dt, x2, dA, iA[J]);
    h[J] = __builtin_fmaf(dA, h[J], k * (u * row_bcast<J>(bc)));
    if constexpr (J == 0) y = row_bcast<NS>(bc) * h[0];
    else fmac_row_bcast<NS + J>(y, bc, h[J]);
    state_step_zoh<NS, J + 1>(h, A2, iA, dt, u, bc, y);
  }
}

// One step of a lane's two states (eight-lane state split), with the lane's
// own B and C values (b4 = B_0, B_1, C_0, C_1, read from LDS): there are
// eight state groups per wave, so a 16-lane row holds two of them and a row
// broadcast cannot serve both.  With ZOH, dtu is u and the write is k u B.
template <bool ZOH>
__device__ __forceinline__ void state_step2(float (&h)[2], const float (&A2)[2], const float (&iA)[2],
                                            float dt, float dtu, const float4 &b4, float &y) {
  const float x0 = dt * A2[0], x1 = dt * A2[1];
  const float a0 = hw_exp2(x0), a1 = hw_exp2(x1);
  float w0 = dtu * b4.x, w1 = dtu * b4.y;
  if constexpr (ZOH) {
    w0 *= zoh_coef(dt, x0, a0, iA[0]);
    w1 *= zoh_coef(dt, x1, a1, iA[1]);
  }
  h[0] = __builtin_fmaf(a0, h[0], w0);
  h[1] = __builtin_fmaf(a1, h[1], w1);
  y = __builtin_fmaf(b4.w, h[1], b4.z * h[0]);
}

// Calls f(std::integral_constant<int, I>()) for I = 0 .. N-1 in order.
template <typename F, int... I>
__device__ __forceinline__ void for_slots_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void for_slots(F &&f) {
  for_slots_impl(f, std::make_integer_sequence<int, N>());
}

// Workgroup barrier that orders LDS only: global loads issued before it stay
// in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave's LDS area.  The staging side (PREP, BC and the conv rows CX) is
// live from a tile's staging to its read-back into registers; the partial
// sums PART from the scan of a tile to their read in the combine.  In a
// wave's program order these never overlap (scan k, read partials k, stage
// k+1, read back k+1), so PART shares the area's start with PREP.
// With the eight-lane state split (R = 8) the scan reads B and C from LDS
// step by step while it writes its partials, so PART gets its own place.
template <int T, int R, bool CV>
struct Layout {
  static constexpr int PSTR = 2 * T + 2;                  // (dt, dt u) per row; PSTR/2 odd
  static constexpr int QSTR = T + 1;                      // partials per lane, odd
  static constexpr int PREP = R * PSTR;
  static constexpr int BC = 32 * T;                       // per step: B 0..15, C 16..31 (R = 8:
                                                          // per state pair n/2, B B C C)
  static constexpr int PART = 64 * QSTR;
  static constexpr int XH = T + 4;                        // conv input row: 3 halo, T, 1 spare
  static constexpr int CX = CV ? R * XH : 0;
  static constexpr int STAGE = PREP + BC + CX;
  static constexpr bool OVERLAY = R != 8;
  static constexpr int PART_AT = OVERLAY ? 0 : (STAGE + 3) / 4 * 4;
  static constexpr int WAVE = OVERLAY ? (STAGE > PART ? STAGE : PART) : PART_AT + PART;  // floats per wave
  static_assert(WAVE % 4 == 0 || OVERLAY, "16-byte B/C reads of the second wave stay aligned");
  static_assert(WAVE % 2 == 0, "float2 staging of the second wave stays 8-byte aligned");
};

// Row stride of the LDS exchange block for n parked steps: >= n and
// congruent to T mod 32, so that a combine instruction (T consecutive steps
// of 64/T channels) hits 32 distinct banks.
__host__ __device__ inline int xchg_stride(int64_t n, int T) {
  return static_cast<int>(n + (((T - n) % 32) + 32) % 32);
}

// Register budget: 4 waves per SIMD with 8-step tiles (3 with the fused
// conv, whose weights and carried inputs do not fit 128 VGPRs), 2 with
// 16-step tiles (whose three tiles in flight and staged copies need about
// 190 VGPRs, 240 with the conv), 3 with 16-step tiles and the 8-lane split
// (about 150; 2 with ZOH and the conv together).
// A bidirectional workgroup holds one or two row blocks (DIRS waves each):
// with two, its four waves land on distinct SIMDs and every SIMD of a CU
// carries the same number of waves.
template <typename Tin, int SPLIT, int DIRS, int XMODE, int T, int OPT>
__global__ void __launch_bounds__(DIRS == 2 ? 256 : 64)
__attribute__((amdgpu_waves_per_eu(T == 16 ? (SPLIT == 8 && OPT != (kOptZoh | kOptConv) ? 3 : 2)
                                                     : ((OPT & kOptConv) != 0 ? 3 : 4))))
scan_kernel(const ScanArgs p) {
  constexpr bool ZOH = (OPT & kOptZoh) != 0;
  constexpr bool CONV = (OPT & kOptConv) != 0;
  constexpr bool CK = (OPT & kOptBwdPrep) != 0;  // prepare the backward pass (checkpoints, gate)
  constexpr bool CKS = CK || (OPT & kOptCk) != 0; // store the backward's checkpoints
  constexpr int NS = 16 / SPLIT;                 // states per lane
  constexpr int R = 64 / SPLIT;                  // channels per workgroup
  constexpr int PE = R * T / 64;                 // staged (dt, u) elements per lane per tile
  constexpr int BQ = T / 4;                      // B (and C) loads per lane per tile
  constexpr uint32_t ES = sizeof(Tin);
  constexpr int NB = 3;                          // tiles in flight (prefetch distance)
  using Lay = Layout<T, R, CONV>;
  static_assert(((NS >= 4 && NS <= 8 && R % 16 == 0) || (NS == 2 && R == 8)) && T % 4 == 0 &&
                    (R * T) % 64 == 0, "shape");
  static_assert(DIRS == 1 ? XMODE == kXNone : XMODE != kXNone, "mode");
  static_assert(!CK || (T == kBwdTile && XMODE == kXLds), "gate backward: the on-chip exchange");
  static_assert(!CKS || T == kBwdTile || T == 2 * kBwdTile, "checkpoints: at the backward's 8-step tiles");

  // Workgroups dispatched after the first round (every CU full) start beside
  // older waves, which the SIMD's oldest-first issue favours; a higher wave
  // priority lets them catch up, so that the SIMDs run out of work closer
  // together (a shorter tail of SIMDs with one or two waves left).  Measured
  // with the on-chip exchange (1.5 rounds at the Vim-T shape: about 1.5 %
  // off the kernel); the long global-exchange scans, three rounds and more,
  // lost 0.5 % with it.
  if constexpr (XMODE == kXLds) {
    if (static_cast<int>(blockIdx.x) >= p.prio_from) __builtin_amdgcn_s_setprio(2);
  }
  extern __shared__ float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsub = static_cast<int>(blockDim.x) / (64 * DIRS);   // row blocks per workgroup
  const int sub = wave / DIRS;                   // row block within the workgroup
  const int dw = wave - sub * DIRS;              // direction wave of the row block
  const int lane = threadIdx.x & 63;
  const int64_t dim = p.dim;
  const int L = static_cast<int>(p.L);
  const int XS = xchg_stride(L, T);
  float *const sbase = smem + sub * (DIRS * Lay::WAVE + (XMODE == kXLds ? R * XS : 0));
  float *const prep = sbase + dw * Lay::WAVE;    // [R][PSTR]
  float *const bcs = prep + Lay::PREP;           // [T][32]
  float *const xs = bcs + Lay::BC;               // [R][XH] conv input (CONV)
  float *const part = prep + Lay::PART_AT;       // [64 lanes][QSTR], shares the staging area (R > 8)
  float *const xlds = sbase + DIRS * Lay::WAVE;  // [R][XS]   (kXLds)

  const int sp = lane / R;                       // state group
  const int r = lane % R;                        // channel within the block
  const bool rev = DIRS == 2 ? dw == 1 : p.reverse != 0;
  const bool fwd_wave = DIRS == 2 && dw == 0;

  // Row block blk = (batch row b, channels d0 ..).  A workgroup's last row
  // blocks may lie past the end: they get no rows, so every access of theirs
  // is out of range, and they still take part in the barriers.
  const int nrb = static_cast<int>((dim + R - 1) / R);
  const int blk_all = xcd_remap(blockIdx.x, gridDim.x) * nsub + sub;
  const bool valid = blk_all < p.batch * nrb;
  const int blk = valid ? blk_all : 0;
  const int b = blk / nrb;
  const int d0 = (blk - b * nrb) * R;
  const int rows = valid ? static_cast<int>(dim - d0 < R ? dim - d0 : R) : 0;
  const int nt = (L + T - 1) / T;
  const int half = (nt + 1) / 2;                 // forward wave's first-visit tiles
  const int dstate = p.dstate;
  const bool gated = p.z != nullptr;

  // Resources: the block's [rows x L] slab of each token tensor (rows past
  // dim are out of range), one batch row of B and C, the block's exchange
  // rows (kXGlobal).
  const DirPtrs P = p.dir[DIRS == 2 ? dw : 0];
  const int64_t rowbase = (static_cast<int64_t>(b) * dim + d0) * L;
  const uint32_t slab = static_cast<uint32_t>(rows) * static_cast<uint32_t>(L) * ES;
  const Rsrc rU = make_rsrc(static_cast<const Tin *>(P.u) + rowbase, slab);
  const Rsrc rD = make_rsrc(static_cast<const Tin *>(P.delta) + rowbase, slab);
  const Rsrc rZ = make_rsrc(gated ? static_cast<const Tin *>(p.z) + rowbase : nullptr, gated ? slab : 0);
  const Rsrc rO = make_rsrc(static_cast<Tin *>(p.out) + rowbase, slab);
  const uint32_t bcext = valid ? (static_cast<uint32_t>(dstate - 1) * static_cast<uint32_t>(P.bsn) +
                                  static_cast<uint32_t>(L - 1) * static_cast<uint32_t>(P.bst) + 1) * ES
                                : 0u;
  const Rsrc rB = make_rsrc(static_cast<const Tin *>(P.B) + static_cast<int64_t>(b) * P.bsb, bcext);
  const Rsrc rC = make_rsrc(static_cast<const Tin *>(P.C) + static_cast<int64_t>(b) * P.bsb, bcext);
  const uint32_t xstride = static_cast<uint32_t>(p.xstride);
  float *const xrow = XMODE == kXGlobal ? p.xglobal + (static_cast<int64_t>(b) * dim + d0) * p.xstride
                                        : nullptr;
  const uint32_t xbytes = static_cast<uint32_t>(rows) * xstride * 4u;
  const Rsrc rX = make_rsrc(xrow, XMODE == kXGlobal ? xbytes : 0u);

  // ---- scan role: channel d0 + r, states n0 .. n0 + NS - 1 (states at or
  // beyond dstate have A = 0 and zero B/C, so they stay at zero)
  // Parameters are read through resources too (rows past dim and states past
  // dstate read 0), so that all of them are in flight at once with the first
  // tiles instead of one load round trip after another.
  const int n0 = sp * NS;
  const Rsrc rA = make_rsrc(P.A + static_cast<int64_t>(d0) * dstate,
                            static_cast<uint32_t>(rows * dstate) * 4u);
  const Rsrc rDp = make_rsrc(P.D + d0, static_cast<uint32_t>(rows) * 4u);
  const Rsrc rBias = make_rsrc(P.bias != nullptr ? P.bias + d0 : nullptr,
                               P.bias != nullptr ? static_cast<uint32_t>(rows) * 4u : 0u);
  const Rsrc rCw = make_rsrc(CONV ? P.cw + static_cast<int64_t>(d0) * 4 : nullptr,
                             CONV ? static_cast<uint32_t>(rows) * 16u : 0u);
  const Rsrc rCb = make_rsrc(CONV && P.cb != nullptr ? P.cb + d0 : nullptr,
                             CONV && P.cb != nullptr ? static_cast<uint32_t>(rows) * 4u : 0u);
  // Backward preparation (CK): the state entering each tile, as the backward
  // kernel's first pass would store it, and the gate's backward in place of
  // out.  Checkpoints are tile-major per row block, [tile][16 channels][16
  // states], so that a wave's checkpoints of one tile are one contiguous
  // kilobyte (a row block past the end has none; channels past dim store
  // zeros).
  // With 16-step tiles a checkpoint goes out at visit positions 0 and 8; with
  // the 8-lane split a wave fills half of a 16-channel block.
  const int nt8 = (L + kBwdTile - 1) / kBwdTile;
  const int nrb16 = static_cast<int>((dim + 15) / 16);
  const Rsrc rCk = make_rsrc(CKS ? p.ck[dw] + (static_cast<int64_t>(b) * nrb16 + d0 / 16) * nt8 * 256 : nullptr,
                             CKS && valid ? static_cast<uint32_t>(nt8) * 1024u : 0u);
  const uint32_t ck_lane = static_cast<uint32_t>((d0 % 16 + r) * 16 + sp * NS) * 4u;

  const Rsrc rGz = make_rsrc(CK ? p.gz + rowbase : nullptr, CK ? slab : 0u);
  const Rsrc rDo = make_rsrc(CK ? p.dout + rowbase : nullptr, CK ? slab : 0u);
  const Rsrc rDy = make_rsrc(CK ? p.dy + (static_cast<int64_t>(b) * nrb + d0 / R) * nt * 16 * T : nullptr,
                             CK && valid ? static_cast<uint32_t>(nt * 16 * T) * 4u : 0u);
  const Rsrc rDz = make_rsrc(CK ? p.dz + rowbase : nullptr, CK ? slab : 0u);
  float A2[NS], iA[NS], h[NS];
  auto store_ck = [&](int tile8) __attribute__((always_inline)) {
    if constexpr (NS == 4) bstore4(rCk, ck_lane + static_cast<uint32_t>(tile8) * 1024u, h);
    else if constexpr (NS == 2) bstore2(rCk, ck_lane + static_cast<uint32_t>(tile8) * 1024u, h);
  };
#pragma unroll
  for (int j = 0; j < NS; ++j) h[j] = 0.0f;
  // lane j of each 16-lane row holds B[n0 + j] (j < NS) or C[n0 + j - NS]
  const int rl = lane & 15;
  const int bc_slot = rl < NS ? n0 + rl : (rl < 2 * NS ? 16 + n0 + rl - NS : 0);

  // ---- staging role.  Element e = lane + 64 i of the R x T tile is (row
  // srow_i = e / T, visit position sq = e % T); every element of a lane has
  // the same sq, hence the same step offset tq within its tile (sq forward,
  // T-1-sq backward): step t = jT + tq of tile j.  Per element: the byte
  // offset of its step in tile 0 (rows past dim are past the slab), its
  // exchange offsets and its bias.
  const int sq = lane % T;
  const int tq = rev ? T - 1 - sq : sq;
  int srow[PE];
  uint32_t ob[PE], oxl[PE], oxg[PE];
  float sbias[PE], sD[PE];
  // Conv (CONV): the element's weights and bias, its raw input of the
  // previous tile, and where that value goes: the halo slot (visit position
  // T-3+h of the previous tile, stored at h) for the last three positions,
  // else the row's spare slot.
  float cw[PE][4], cb[PE], xprev[PE];
  int hx[PE];
  float ukeep[PE];                               // u of the staged tile, for its D u skip
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    srow[i] = lane / T + i * (64 / T);
    ob[i] = (static_cast<uint32_t>(srow[i]) * static_cast<uint32_t>(L) + tq) * ES;
    oxl[i] = static_cast<uint32_t>(srow[i] * XS + tq);
    oxg[i] = (static_cast<uint32_t>(srow[i]) * xstride + tq) * 4u;
    xprev[i] = 0.0f;                             // zero padding before the first step
    hx[i] = srow[i] * Lay::XH + (sq >= T - 3 ? sq - (T - 3) : T + 3);
  }
  // B and C: load i of a lane covers visit position q = lane / 16 + 4 i and
  // state n = lane % 16 (past dstate: out of range, so it stages 0).
  const int n_bc = lane % 16;
  uint32_t bo[BQ];
#pragma unroll
  for (int i = 0; i < BQ; ++i) {
    const int q = lane / 16 + 4 * i;
    const int qt = rev ? T - 1 - q : q;
    bo[i] = n_bc < dstate ? (static_cast<uint32_t>(n_bc) * static_cast<uint32_t>(P.bsn) +
                             static_cast<uint32_t>(qt) * static_cast<uint32_t>(P.bst)) * ES
                          : kOob;
  }
  const uint32_t bst_bytes = static_cast<uint32_t>(P.bst) * ES;

  auto tile_of = [&](int k) __attribute__((always_inline)) { return rev ? nt - 1 - k : k; };
  // Byte offset of element i in tile j (jT = j T), or out of range for steps past L.
  auto tok_off = [&](int i, int jT, bool in_seq) __attribute__((always_inline)) {
    return pin_u(in_seq ? ob[i] + static_cast<uint32_t>(jT) * ES : kOob);
  };

  // Raw global values of NB tiles in flight (tile m in slot m % NB).
  // Nothing reads them before the tile is staged: with a static count of
  // loads in flight, the wait for an older tile leaves the later prefetches
  // in flight.
  float ru[NB][PE], rd[NB][PE], rb[NB][BQ], rc[NB][BQ];

  // Steps past L must stage u = 0 only where they come before real steps
  // of the visit: in the first tile of a reversed visit, which the prologue
  // loads.  Later tiles take the plain offsets: past L the slab's last row
  // reads 0 (its offsets leave the slab), the others the next row's values,
  // which only feed states after the last real step and outputs that land
  // in the exchange rows' padding or are masked at the store.
  auto stage_load = [&](int k, auto par, auto masked) __attribute__((always_inline)) {
    constexpr int Q = decltype(par)::value;
    const int jT = tile_of(k) * T;
    const bool in_seq = !decltype(masked)::value || tq < L - jT;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const uint32_t o = tok_off(i, jT, in_seq);
      ru[Q][i] = bload<Tin>(rU, o);
      rd[Q][i] = bload<Tin>(rD, o);
    }
    const uint32_t tb = static_cast<uint32_t>(jT) * bst_bytes;
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      rb[Q][i] = bload<Tin>(rB, bo[i] + tb);
      rc[Q][i] = bload<Tin>(rC, bo[i] + tb);
    }
  };

  // Stages (dt, dt u) for the scan ((dt, u) with the zero-order hold), for
  // tile kt, and keeps u in registers for the skip term.  Steps past L
  // and channels past dim stage u = 0, so the state only decays where it is
  // zero (before the first real step) or no longer read; states past dstate
  // stage B = C = 0.
  // CONV: the loaded values are the conv input x.  The wave writes the
  // tile's x (row slots 3..T+2, in visit order) and the previous tile's last
  // three (slots 0..2), then reads each element's three predecessors back:
  // u = SiLU(cb + w0 x[-3] + w1 x[-2] + w2 x[-1] + w3 x[0]); the reads
  // follow the other lanes' writes (wave_lds_fence).
  auto stage_store = [&](auto par, int kt) __attribute__((always_inline)) {
    constexpr int Q = decltype(par)::value;
    const bool sp_on = p.softplus != 0;
    float uin[PE];
    if constexpr (CONV) {
      float xc[PE];
#pragma unroll
      for (int i = 0; i < PE; ++i) {
        xc[i] = pin(ru[Q][i]);
        xs[hx[i]] = xprev[i];
        xs[srow[i] * Lay::XH + 3 + sq] = xc[i];
        xprev[i] = xc[i];
      }
      wave_lds_fence();
      const bool in_seq = tq < L - tile_of(kt) * T;
#pragma unroll
      for (int i = 0; i < PE; ++i) {
        const float *const xr = xs + srow[i] * Lay::XH + sq;
        float v = __builtin_fmaf(cw[i][3], xc[i], cb[i]);
        v = __builtin_fmaf(cw[i][2], xr[2], v);
        v = __builtin_fmaf(cw[i][1], xr[1], v);
        v = __builtin_fmaf(cw[i][0], xr[0], v);
        uin[i] = in_seq ? silu_f(v) : 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PE; ++i) uin[i] = pin(ru[Q][i]);
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const float x = pin(rd[Q][i]) + sbias[i];
      const float uv = uin[i];
      const float dtv = sp_on ? softplus_f(x) : x;
      *reinterpret_cast<float2 *>(prep + srow[i] * Lay::PSTR + 2 * sq) =
          make_float2(dtv, ZOH ? uv : dtv * uv);
      ukeep[i] = uv;
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      float *const q = bcs + (lane / 16 + 4 * i) * 32 + (NS == 2 ? (n_bc >> 1) * 4 + (n_bc & 1) : n_bc);
      q[0] = pin(rb[Q][i]);
      q[NS == 2 ? 2 : 16] = pin(rc[Q][i]);
    }
  };

  // The staged tile is read back into registers right after it is staged, so
  // the LDS latency overlaps the finishing work of the previous tile.
  const float *const pr_lane = prep + r * Lay::PSTR;
  const float *const bc_lane = bcs + bc_slot;
  float *const part_lane = part + lane * Lay::QSTR;
  float2 dus[T];
  float bcv[T];
  auto read_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < T; ++q) {
      dus[q] = *reinterpret_cast<const float2 *>(pr_lane + 2 * q);
      if constexpr (NS != 2) bcv[q] = bc_lane[q * 32];
    }
  };

  // (two-state split: B and C of the lane's state pair, read step by step)
  const float *const b4_lane = bcs + 4 * sp;
  auto do_scan = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < T; ++q) {
      if constexpr (CKS && T == 2 * kBwdTile) {
        // the state entering 8-step tile 2 j + (q / 8) (visit order reversed
        // within a backward 16-step tile; past the last 8-step tile: dropped)
        if (q % kBwdTile == 0) store_ck(2 * tile_of(k) + (rev ? 1 - q / kBwdTile : q / kBwdTile));
      }
      float y;
      if constexpr (NS == 2)
        state_step2<ZOH>(h, A2, iA, dus[q].x, dus[q].y, *reinterpret_cast<const float4 *>(b4_lane + q * 32), y);
      else if constexpr (ZOH) state_step_zoh<NS, 0>(h, A2, iA, dus[q].x, dus[q].y, bcv[q], y);
      else state_step<NS, 0>(h, A2, dus[q].x, dus[q].y, bcv[q], y);
      part_lane[q] = y;
    }
  };

  // Finishing a tile: its SPLIT partial sums and the skip D u per element,
  // plus the gate (one direction; second visits) and the partner's parked
  // sums (second visits).  The global values of tile k are loaded one
  // iteration ahead (slot k % NB), the LDS ones right after the scan.  kXLds
  // parks both waves' first visits in the LDS block [R][XS] and finishes
  // there in place; kXGlobal parks in global memory and finishes into out.
  float zr[NB][PE], xg[NB][PE], xl[PE], uk[PE], ps[PE][SPLIT];
  auto comb_load = [&](int k, auto slot, auto second) __attribute__((always_inline)) {
    constexpr int Q = decltype(slot)::value;
    constexpr bool SECOND = decltype(second)::value;
    const int jT = tile_of(k) * T;
    const bool in_seq = tq < L - jT;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      if (DIRS == 1 || SECOND) zr[Q][i] = bload<Tin>(rZ, tok_off(i, jT, in_seq));
      if (XMODE == kXGlobal && SECOND) xg[Q][i] = bload<float>(rX, oxg[i] + static_cast<uint32_t>(jT) * 4u);
    }
  };
  auto comb_read = [&](int k, auto second) __attribute__((always_inline)) {
    constexpr bool SECOND = decltype(second)::value;
    const int jT = tile_of(k) * T;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
#pragma unroll
      for (int s = 0; s < SPLIT; ++s) ps[i][s] = part[(s * R + srow[i]) * Lay::QSTR + sq];
      uk[i] = ukeep[i];
      if (XMODE == kXLds && SECOND) xl[i] = xlds[oxl[i] + jT];
    }
  };
  auto do_combine = [&](int k, auto slot, auto second) __attribute__((always_inline)) {
    constexpr int Q = decltype(slot)::value;
    constexpr bool SECOND = decltype(second)::value;
    const int jT = tile_of(k) * T;
    const bool in_seq = tq < L - jT;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      float y = ps[i][0];
#pragma unroll
      for (int s = 1; s < SPLIT; ++s) y += ps[i][s];
      y = __builtin_fmaf(sD[i], uk[i], y);
      if (DIRS == 1 || SECOND) {
        const float g = gated ? silu_f(pin(zr[Q][i])) : 1.0f;
        const float other = XMODE == kXLds ? xl[i] : XMODE == kXGlobal ? pin(xg[Q][i]) : 0.0f;
        const float v = DIRS == 1 ? y * g : p.scale * (other + y) * g;
        // rows past dim and steps past L: out of range, or the LDS block's padding
        if (XMODE == kXLds) xlds[oxl[i] + jT] = v;
        else bstore<Tin>(rO, tok_off(i, jT, in_seq), v);
      } else if (XMODE == kXLds) {
        xlds[oxl[i] + jT] = y;
      } else {
        bstore<float>(rX, oxg[i] + static_cast<uint32_t>(jT) * 4u, y);
      }
    }
  };

  using First = std::integral_constant<bool, false>;
  using Second = std::integral_constant<bool, true>;

  // One iteration k (slot Q = k % NB): finishing loads of k+1, prefetch of
  // tile k+NB into the slot tile k has left, scan k, partial reads of k,
  // stage and read back k+1, combine k.  Each hand-over of LDS data between
  // lanes of the wave is ordered by wave_lds_fence (no barrier: only this
  // wave touches its area).  The prefetch and the
  // staging run on every iteration (past the end they repeat the last tile,
  // whose staged copy is never scanned): a load issued under a branch would
  // make the count of loads in flight path-dependent.
  auto iteration = [&](int k, auto slot, auto second) __attribute__((always_inline)) {
    using Qn = std::integral_constant<int, (decltype(slot)::value + 1) % NB>;
    comb_load(k + 1 < nt ? k + 1 : nt - 1, Qn(), second);
    stage_load(k + NB < nt ? k + NB : nt - 1, slot, std::false_type());
    if constexpr (CKS && T == kBwdTile) store_ck(tile_of(k));
    wave_lds_fence();                    // staged tile k read back before its partials overwrite it
    do_scan(k);
    wave_lds_fence();
    comb_read(k, second);
    wave_lds_fence();
    stage_store(Qn(), k + 1 < nt ? k + 1 : nt - 1);
    wave_lds_fence();
    read_tile();
    do_combine(k, slot, second);
  };
  // Iterations k0 .. k1-1 of one phase, unrolled NB times so that every
  // slot index is a compile-time constant.
  auto run = [&](int k0, int k1, auto second) __attribute__((always_inline)) {
    int k = k0;
    for_slots<NB>([&](auto s) __attribute__((always_inline)) {       // up to a multiple of NB
      if (decltype(s)::value > 0 && k < k1 && k % NB == decltype(s)::value) iteration(k++, s, second);
    });
    for (; k + NB <= k1; k += NB)
      for_slots<NB>([&](auto s) __attribute__((always_inline)) { iteration(k + decltype(s)::value, s, second); });
    for_slots<NB>([&](auto s) __attribute__((always_inline)) {       // the rest
      if (decltype(s)::value < NB - 1 && k < k1) iteration(k++, s, second);
    });
  };

  // First tiles, then the parameters, all in flight together.
  for_slots<NB>([&](auto s) __attribute__((always_inline)) {
    stage_load(decltype(s)::value < nt ? decltype(s)::value : nt - 1, s, std::true_type());
  });
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n0 + j;
    A2[j] = bload<float>(rA, n < dstate ? static_cast<uint32_t>(r * dstate + n) * 4u : kOob);
  }
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    sbias[i] = bload<float>(rBias, static_cast<uint32_t>(srow[i]) * 4u);
    sD[i] = bload<float>(rDp, static_cast<uint32_t>(srow[i]) * 4u);
    if constexpr (CONV) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        cw[i][k] = bload<float>(rCw, static_cast<uint32_t>(srow[i] * 4 + k) * 4u);
      cb[i] = bload<float>(rCb, static_cast<uint32_t>(srow[i]) * 4u);
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float a = pin(A2[j]);
    if constexpr (ZOH) iA[j] = a != 0.0f ? 1.0f / a : 0.0f;
    A2[j] = a * kLog2e;
  }
  stage_store(std::integral_constant<int, 0>(), 0);
  wave_lds_fence();
  read_tile();
  if (DIRS == 1) {
    comb_load(0, std::integral_constant<int, 0>(), First());
    run(0, nt, First());
    return;
  }

  // Phase 1 has the forward wave on the first ceil(nt/2) tiles and the
  // backward wave on the rest (first visits, parked); after the barrier each
  // wave finishes its remaining tiles against the other's parked sums and
  // writes the output.
  const int n1 = fwd_wave ? half : nt - half;
  run(0, n1, First());
  if (XMODE == kXLds) lds_barrier();
  else __syncthreads();
  // finishing loads of the first second-phase tile (slot n1 % NB)
  for_slots<NB>([&](auto s) __attribute__((always_inline)) {
    if (n1 < nt && n1 % NB == decltype(s)::value) comb_load(n1, s, Second());
  });
  run(n1, nt, Second());

  // ---- short sequences: the block's [rows x L] slab of out is complete in
  // LDS (scaled and gated); write it out with coalesced stores.  With the
  // backward preparation each element also loads z and dout, in flat order:
  // 16 elements per thread per pass keep those loads in flight together
  // (the scan's registers are free by now).  (Done here rather than per tile
  // in the scan loop, whose issue slots the extra exponentials would take.)
  if (XMODE == kXLds && !CK) {
    // Row by row (rows are consecutive in out, L values each): thread tid
    // takes steps tid + c NT of every row, so the addresses are a lane
    // offset per pass plus a per-row constant (an LDS immediate, a scalar
    // store offset).
    lds_barrier();
    constexpr int NT = 64 * DIRS;
    const int tid = static_cast<int>(threadIdx.x) - sub * NT;
    for (int t0 = 0; t0 < L; t0 += NT) {     // uniform passes
      const int t = t0 + tid;
      const bool in = t < L;
      const uint32_t o = in ? static_cast<uint32_t>(t) * ES : kOob;
      const float *const xc = xlds + (in ? t : 0);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        if (rr < rows)
          bstore_s<Tin>(rO, o, static_cast<uint32_t>(rr) * static_cast<uint32_t>(L) * ES, xc[rr * XS]);
      }
    }
  } else if (XMODE == kXLds) {
    lds_barrier();
    constexpr int NT = 64 * DIRS, U = CK ? 16 : 4;
    const int n = rows * L;
    const int tid = static_cast<int>(threadIdx.x) - sub * NT;
    int fr = tid / L, ft = tid % L;
    for (int f0 = tid; f0 < n; f0 += U * NT) {
      float v[U], gzv[U], gdo[U];
      uint32_t oty[U];                       // (CK) tile-major offset of dy
#pragma unroll
      for (int u = 0; u < U; ++u) {          // reads first, so their latency overlaps
        v[u] = xlds[(fr < R ? fr : R - 1) * XS + ft];
        if constexpr (CK) oty[u] = static_cast<uint32_t>(((ft / T) * 16 + fr) * T + ft % T) * 4u;
        ft += NT;
        while (ft >= L) { ft -= L; ++fr; }
        if constexpr (CK) {
          const int f = f0 + u * NT;
          const uint32_t o = pin_u(f < n ? static_cast<uint32_t>(f) * 4u : kOob);
          gzv[u] = bload<float>(rGz, o);
          gdo[u] = bload<float>(rDo, o);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * NT;
        if constexpr (CK) {
          // v is the ungated y: dy = s dout SiLU(z), dz = s dout y SiLU'(z),
          // SiLU'(z) = sg (1 + z (1 - sg)), sg = sigmoid(z)
          const uint32_t o = pin_u(f < n ? static_cast<uint32_t>(f) * 4u : kOob);
          const float zv = pin(gzv[u]);
          const float g = p.gscale * pin(gdo[u]);
          const float sg = hw_rcp(1.0f + hw_exp2(-zv * kLog2e));
          bstore<float>(rDy, f < n ? oty[u] : kOob, g * zv * sg);
          bstore<float>(rDz, o, g * v[u] * (sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f)));
        } else {
          bstore<Tin>(rO, pin_u(f < n ? static_cast<uint32_t>(f) * ES : kOob), v[u]);
        }
      }
    }
  }
}

template <typename Tin, int SPLIT, int DIRS, int XMODE, int T, int OPT>
hipError_t launch_one(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  auto kern = scan_kernel<Tin, SPLIT, DIRS, XMODE, T, OPT>;
  static bool attr_set = false;  // benign race: the attribute value is idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // the first round: resident workgroups per CU times the CUs
  ScanArgs args = a;
  args.prio_from = INT_MAX;
  int dev = 0, per_cu = 0;
  static int cus[64] = {};           // per device; benign race (the same value)
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    if (cus[dev] == 0) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
    }
    if (cus[dev] > 0 &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), plan.threads,
                                                     plan.lds) == hipSuccess &&
        per_cu > 0 && static_cast<int64_t>(per_cu) * cus[dev] < plan.blocks)
      args.prio_from = per_cu * cus[dev];
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(plan.blocks)), dim3(plan.threads), plan.lds,
                     s, args);
  return hipGetLastError();
}

template <typename Tin, int SPLIT, int OPT>
hipError_t dispatch_mode(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (plan.dirs == 1) return launch_one<Tin, SPLIT, 1, kXNone, 16, OPT>(plan, a, s);
  if (plan.xmode == kXLds) return launch_one<Tin, SPLIT, 2, kXLds, 8, OPT>(plan, a, s);
  if (plan.S == 8) return launch_one<Tin, 8, 2, kXGlobal, 16, OPT>(plan, a, s);
  return launch_one<Tin, SPLIT, 2, kXGlobal, 16, OPT>(plan, a, s);
}

template <typename Tin>
hipError_t dispatch_dtype(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
  if (a.ck[0] != nullptr) {
    // backward preparation: fp32, both directions, no conv; the gate's
    // backward too (dy set) on the on-chip exchange, else checkpoints only
    if constexpr (std::is_same<Tin, float>::value) {
      if (plan.dirs == 2 && !a.conv && a.dy != nullptr && plan.xmode == kXLds)
        return a.zoh ? launch_one<float, 4, 2, kXLds, 8, kOptBwdPrep | kOptZoh>(plan, a, s)
                     : launch_one<float, 4, 2, kXLds, 8, kOptBwdPrep>(plan, a, s);
      if (plan.dirs == 2 && !a.conv && a.dy == nullptr) {
        if (plan.xmode == kXLds)
          return a.zoh ? launch_one<float, 4, 2, kXLds, 8, kOptCk | kOptZoh>(plan, a, s)
                       : launch_one<float, 4, 2, kXLds, 8, kOptCk>(plan, a, s);
        if (plan.S == 8)
          return a.zoh ? launch_one<float, 8, 2, kXGlobal, 16, kOptCk | kOptZoh>(plan, a, s)
                       : launch_one<float, 8, 2, kXGlobal, 16, kOptCk>(plan, a, s);
        return a.zoh ? launch_one<float, 4, 2, kXGlobal, 16, kOptCk | kOptZoh>(plan, a, s)
                     : launch_one<float, 4, 2, kXGlobal, 16, kOptCk>(plan, a, s);
      }
    }
    return hipErrorInvalidValue;
  }
  switch ((a.zoh ? kOptZoh : 0) | (a.conv ? kOptConv : 0)) {
    case 0: return dispatch_mode<Tin, 4, 0>(plan, a, s);
    case kOptZoh: return dispatch_mode<Tin, 4, kOptZoh>(plan, a, s);
    case kOptConv: return dispatch_mode<Tin, 4, kOptConv>(plan, a, s);
    default: return dispatch_mode<Tin, 4, kOptZoh | kOptConv>(plan, a, s);
  }
}

size_t lds_bytes(int split, int dirs, int T, int xmode, int64_t L, bool conv) {
  const int R = 64 / split;
  const size_t stage = R * (2 * T + 2) + 32 * T + (conv ? R * (T + 4) : 0);   // Layout::STAGE
  const size_t part = 64 * (T + 1);                                            // Layout::PART
  const size_t wave = R != 8 ? (stage > part ? stage : part) : (stage + 3) / 4 * 4 + part;
  size_t f = static_cast<size_t>(dirs) * wave;
  if (xmode == kXLds) f += static_cast<size_t>(R) * xchg_stride(L, T);
  return f * sizeof(float);
}

}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t L, int dstate, int dirs, bool conv) {
  (void)dstate;
  ScanPlan pl{};
  pl.dirs = dirs;
  // Each channel's 16 states are split over 4 lanes: a two-lane split needs
  // fewer instructions per state but leaves half the waves, and measured
  // slower on every workload tried (fewer waves to hide latency, and a
  // larger LDS exchange per workgroup).  Long bidirectional sequences with
  // fewer than two waves per SIMD (1024 SIMDs) split over 8 lanes instead:
  // a wave alone on a SIMD issues about one instruction per 5 cycles, two
  // or more share it at about 2.2 each, so twice the waves with 60 % of the
  // instructions each finish sooner.
  pl.S = 4;
  pl.threads = 64 * dirs;
  int64_t nblk = batch * ((dim + 64 / pl.S - 1) / (64 / pl.S));
  // Tile length: 16 steps where the registers allow it (one direction, or
  // the global exchange: longer row segments per load and half the per-tile
  // overhead); 8 for the on-chip exchange, whose LDS footprint grows with T.
  pl.sub = 1;
  pl.chunks = 1;
  pl.chunk_len = static_cast<int>(L);
  if (dirs == 1) {
    pl.T = 16;
    pl.xmode = kXNone;
    // Few row blocks (at most 256, a quarter of a wave per SIMD): the
    // sequence-parallel kernel, one workgroup of four waves per channel,
    // each lane on a sub-chunk of ceil(L / 64) steps, the row staged in LDS
    // (L <= 256).  It does about twice the arithmetic, which pays only where
    // SIMDs would otherwise sit idle, and only for sequences long enough to
    // split.
    if (nblk <= 256 && L >= 32 && L <= 256) {
      pl.chunks = 64;
      pl.chunk_len = static_cast<int>((L + 63) / 64);
      pl.threads = 256;
      pl.blocks = batch * dim;
      pl.lds = 0;
      return pl;
    }
  } else {
    // On-chip exchange while a row block's area lets four of them share a
    // CU's 160 KB LDS.
    pl.xmode = lds_bytes(pl.S, 2, 8, kXLds, L, conv) <= 40 * 1024 ? kXLds : kXGlobal;
    pl.T = pl.xmode == kXLds ? 8 : 16;
    if (pl.xmode == kXGlobal && nblk * 2 < 2048) {
      pl.S = 8;
      nblk = batch * ((dim + 7) / 8);
    }
    // Two row blocks per workgroup where there are enough of them to give
    // every CU several workgroups: the balanced SIMDs measured 4 % faster on
    // the Vim-T step.  Fewer, larger workgroups would leave CUs idle on small
    // problems; the global exchange measured 1 % slower with two.
    if (pl.xmode == kXLds && nblk >= 2048) pl.sub = 2;
  }
  pl.threads *= pl.sub;
  pl.blocks = (nblk + pl.sub - 1) / pl.sub;
  pl.lds = static_cast<size_t>(pl.sub) * lds_bytes(pl.S, dirs, pl.T, pl.xmode, L, conv);
  return pl;
}

int64_t xchg_global_stride(int64_t L) { return (L + 31) / 32 * 32; }

// The kernel addresses a workgroup's rows, a batch row of B and C, and its
// exchange rows through buffer resources with byte offsets below 2^31
// (offsets may run one tile past the data).
bool scan_offsets_fit(const ScanPlan &plan, const ScanArgs &a, bool bf16) {
  const uint64_t lim = uint64_t{1} << 31;
  const uint64_t es = bf16 ? 2 : 4;
  const uint64_t R = 64 / plan.S;
  const uint64_t Lt = static_cast<uint64_t>(a.L) + plan.T;
  if (R * Lt * es >= lim) return false;
  for (int k = 0; k < plan.dirs; ++k) {
    const DirPtrs &d = a.dir[k];
    const uint64_t ext = static_cast<uint64_t>(a.dstate - 1) * static_cast<uint64_t>(d.bsn) +
                         Lt * static_cast<uint64_t>(d.bst) + 1;
    if (ext * es >= lim) return false;
  }
  if (plan.xmode == kXGlobal && R * static_cast<uint64_t>(a.xstride) * 4 >= lim) return false;
  return true;
}

hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &args, bool bf16, hipStream_t s) {
  if (plan.blocks <= 0) return hipSuccess;
  if (plan.chunks > 1) return launch_scan_chunked(plan, args, bf16, s);
  return bf16 ? dispatch_dtype<bf16_t>(plan, args, s) : dispatch_dtype<float>(plan, args, s);
}

}  // namespace vmk
