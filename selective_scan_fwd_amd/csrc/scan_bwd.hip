// Backward pass of the selective scan (one direction, fp32) for gfx950.
//
// Forward (Vision Mamba page, "A state retains, writes, and reads"): per
// channel, from h = 0, h_t = a_t h_{t-1} + dt_t B_t u_t with a_t = exp(dt_t A),
// y_t = sum_n C_t h_t + D u_t, dt = softplus(delta + bias).  Given dy = dL/dy,
// the adjoint of the state runs against the visit order:
//   g_t = C_t dy_t + a_{t+1} g_{t+1}                     (g = dL/dh_t)
// and the gradients collect along it:
//   dC_t += dy_t h_t          dB_t += g_t dt_t u_t       (summed over channels)
//   dA   += g_t a_t h_{t-1} dt_t                          (summed over batch)
//   du_t  = dt_t sum_n g_t B_t + D dy_t
//   ddt_t = u_t sum_n g_t B_t + sum_n g_t a_t h_{t-1} A
//   ddelta_t = ddt_t sigmoid(delta_t + bias) (softplus), dbias, dD summed.
// a_t h_{t-1} is formed as a product from the kept states (the tile's
// checkpoint for its first step), not as h_t - dt_t B_t u_t, which would
// leave rounding residue where h_{t-1} is exactly zero.
// With the zero-order-hold write (ZOH) the write is k_t B_t u_t with
// k = expm1(dt A) / A per state, so dt u becomes k u in dB and du, and k's
// derivatives join the rest: dk/ddt = a_t and dk/dA (zoh_coef_dA):
//   dA   += g_t (a_t h_{t-1} dt_t + B_t u_t dk/dA)
//   du_t  = sum_n g_t B_t k + D dy_t
//   ddt_t = sum_n g_t a_t (A h_{t-1} + B_t u_t).
//
// Work decomposition: as the forward kernel, one wave covers 16 channels of
// one batch row, a lane holding 4 of a channel's 16 states.  Pass 1 runs the
// state forward over the sequence and stores the state at every tile start
// (checkpoints).  Pass 2 visits the tiles in reverse: it restarts the state
// from the tile's checkpoint, keeps the tile's states and decays in
// registers, then runs the adjoint back through the tile.  Per-channel sums
// (du, ddelta) meet in LDS like the forward's partial sums; the sums over
// channels (dB, dC) are reduced over the wave's 16 channels in LDS and
// written as one partial per channel block; the sums over batch rows (dA, dD,
// dbias) are written as one partial per batch row.  Two small kernels add
// the partials, in a fixed order (deterministic).
#include "scan_device.h"
#include "vm_internal.h"

namespace vmk {
namespace {

constexpr int kNS = 4;                 // states per lane
constexpr int kR = 16;                 // channels per wave

template <int T>
struct BwdLayout {
  static constexpr int PST = 4 * T + 4;               // (dt, dt u, dy, -) per step, per row
  static constexpr int PREP = kR * PST;
  static constexpr int BC = 32 * T;                   // B in slots 0..15, C in 16..31
  static constexpr int STAGE = PREP + BC;
  static constexpr int QSTR = T + 1;
  static constexpr int PART = 2 * 64 * QSTR;          // per-lane sums of g B and g a h A
  // The partial sums share the staging area: a tile's staged values are in
  // registers before its adjoint writes them.
  static constexpr int AREA = STAGE > PART ? STAGE : PART;
  // dC, then dB, contributions [n][q][r].  Row (n, q) starts at
  // (n T + q) RSTR + (n / 4) 16: a lane's 16-byte reads of consecutive rows
  // then fall in distinct banks, and so do the writes of the four 16-lane
  // rows of a wave (state groups n / 4).
  static constexpr int RSTR = kR + 4;
  static constexpr int RED = 16 * T * RSTR + 64;
  // du, ddelta of the last RING_T steps per row (slot t mod RING_T), until
  // their 128-byte lines are complete and go out whole.
  static constexpr int RING_T = 40;
  static constexpr int RING = 2 * kR * RING_T;
  static constexpr int TOTAL = AREA + RED + RING;
};

// The tile's states and decays stay in registers (64 VGPRs with 8-step
// tiles; 4-step tiles fit more workgroups but measured 1.6x slower for their
// per-tile reductions), which sets the register budget at two waves per
// SIMD; the LDS area (under 20 KB, eight waves per CU) does not lower that.
// The ZOH adjoint's extra terms need about 300 registers: one wave per SIMD.
__device__ __forceinline__ const BwdArgs &group_entry(const BwdArgs &a, int) { return a; }
__device__ __forceinline__ const BwdArgs &group_entry(const BwdGroup &g, int k) { return g.a[k]; }

// Arg: BwdArgs (one direction) or BwdGroup (several in one grid).
template <int T, bool ZOH, typename Arg>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ZOH ? 1 : 2)))
scan_bwd_kernel(const Arg arg) {
  using Lay = BwdLayout<T>;
  constexpr int PE = kR * T / 64;      // staged elements per lane per tile
  constexpr int BQ = T / 4;            // B (and C) loads per lane per tile
  extern __shared__ float smem[];
  float *const prep = smem;                       // [R][PST]
  float *const bcs = prep + Lay::PREP;            // [T][32]
  float *const part = smem;                       // [2][64][QSTR], over the staging area
  float *const red = smem + Lay::AREA;            // [16][T][R], padded rows
  float *const ring = red + Lay::RED;             // [2][R][RING_T]
  static_assert(Lay::RING_T % T == 0 && Lay::RING_T >= 32 + T - 1, "ring");

  // a group's grid covers its directions one after another
  const int64_t dim = group_entry(arg, 0).dim;
  const int nrb = static_cast<int>((dim + kR - 1) / kR);
  int blk = xcd_remap(blockIdx.x, gridDim.x), which = 0;
  if constexpr (std::is_same<Arg, BwdGroup>::value) {
    const int nblk = static_cast<int>(arg.a[0].batch) * nrb;
    which = blk / nblk;
    blk -= which * nblk;
  }
  const BwdArgs &p = group_entry(arg, which);

  const int lane = threadIdx.x;
  const int sp = lane / kR, r = lane % kR;
  const bool rev = p.reverse != 0;
  const int L = static_cast<int>(p.L);
  const int b = blk / nrb;
  const int rb = blk - b * nrb;
  const int d0 = rb * kR;
  const int rows = static_cast<int>(dim - d0 < kR ? dim - d0 : kR);
  const int nt = (L + T - 1) / T;
  const int dstate = p.dstate;
  const DirPtrs P = p.dir;

  const int64_t rowbase = (static_cast<int64_t>(b) * dim + d0) * L;
  const uint32_t slab = static_cast<uint32_t>(rows) * static_cast<uint32_t>(L) * 4u;
  const Rsrc rU = make_rsrc(static_cast<const float *>(P.u) + rowbase, slab);
  const Rsrc rDl = make_rsrc(static_cast<const float *>(P.delta) + rowbase, slab);
  const Rsrc rDy = p.dy_tiled ? make_rsrc(p.dy + (static_cast<int64_t>(b) * nrb + rb) * nt * 16 * T,
                                          static_cast<uint32_t>(nt * 16 * T) * 4u)
                             : make_rsrc(p.dy + rowbase, slab);
  const Rsrc rDu = make_rsrc(p.du + rowbase, slab);
  const Rsrc rDd = make_rsrc(p.ddelta + rowbase, slab);
  const uint32_t bcext = (static_cast<uint32_t>(dstate - 1) * static_cast<uint32_t>(P.bsn) +
                          static_cast<uint32_t>(L - 1) * static_cast<uint32_t>(P.bst) + 1) * 4u;
  const Rsrc rB = make_rsrc(static_cast<const float *>(P.B) + static_cast<int64_t>(b) * P.bsb, bcext);
  const Rsrc rC = make_rsrc(static_cast<const float *>(P.C) + static_cast<int64_t>(b) * P.bsb, bcext);
  const Rsrc rA = make_rsrc(P.A + static_cast<int64_t>(d0) * dstate,
                            static_cast<uint32_t>(rows * dstate) * 4u);
  const Rsrc rDp = make_rsrc(P.D + d0, static_cast<uint32_t>(rows) * 4u);
  const Rsrc rBias = make_rsrc(P.bias != nullptr ? P.bias + d0 : nullptr,
                               P.bias != nullptr ? static_cast<uint32_t>(rows) * 4u : 0u);
  // checkpoints of this row block: [tile][16 channels][16 states]
  const Rsrc rCk = make_rsrc(p.ck + (static_cast<int64_t>(b) * nrb + rb) * nt * 256,
                             static_cast<uint32_t>(nt) * 1024u);
  // partial sums over channels of this block: [tile][16 states][T steps]
  // per quantity (positions past L and states past dstate hold zeros)
  const int64_t pbc = (static_cast<int64_t>(rb) * p.batch + b) * nt * 16 * T;
  const uint32_t pbc_bytes = static_cast<uint32_t>(nt * 16 * T) * 4u;
  const Rsrc rPB = make_rsrc(p.pB + pbc, pbc_bytes);
  const Rsrc rPC = make_rsrc(p.pC + pbc, pbc_bytes);

  // ---- state role: channel d0 + r, states n0 .. n0 + 3
  const int n0 = sp * kNS;
  float A2[kNS], An[kNS], iA[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    const int n = n0 + j;
    An[j] = bload<float>(rA, n < dstate ? static_cast<uint32_t>(r * dstate + n) * 4u : kOob);
    A2[j] = An[j] * kLog2e;
    iA[j] = ZOH && An[j] != 0.0f ? 1.0f / An[j] : 0.0f;
  }
  const int rl = lane & 15;
  const int bc_slot = rl < kNS ? n0 + rl : (rl < 2 * kNS ? 16 + n0 + rl - kNS : 0);

  // ---- staging role: element i = (row srow[i], visit position sq)
  const int sq = lane % T;
  const int tq = rev ? T - 1 - sq : sq;
  int srow[PE];
  uint32_t ob[PE], oy[PE];
  float sbias[PE], sD[PE], accD[PE], accB[PE];
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    srow[i] = lane / T + i * (64 / T);
    ob[i] = (static_cast<uint32_t>(srow[i]) * static_cast<uint32_t>(L) + tq) * 4u;
    oy[i] = p.dy_tiled ? static_cast<uint32_t>(srow[i] * T + tq) * 4u : ob[i];
    sbias[i] = bload<float>(rBias, static_cast<uint32_t>(srow[i]) * 4u);
    sD[i] = bload<float>(rDp, static_cast<uint32_t>(srow[i]) * 4u);
    accD[i] = 0.0f;
    accB[i] = 0.0f;
  }
  // Output lines.  A row's element t sits at element offset e0 + row L + t
  // of du (ddelta is taken to share its alignment); line boundaries are where
  // that offset is a multiple of 32.  A tile's du and ddelta go into the ring;
  // every line of a row whose steps are all done then goes out in one burst
  // (a line stored piecewise, one tile apart, is fetched and written back
  // several times).  The ZOH variant, whose registers are tight at one wave
  // per SIMD, stores directly.  A row's items are the lines between its
  // boundaries and the partial lines at its two ends.  Per row (wave-uniform):
  // tb0, its first boundary; the tiles j that complete one of its lines are
  // those with j mod 4 == its class; such an item starts at 8 j + d (visiting
  // backward in t) or ends at 8 j + 1 + d (visiting forward in t, rev).
  static_assert(T == 8, "four tiles per 128-byte line");
  const uint32_t e0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p.du) >> 2) +
                      static_cast<uint32_t>(rowbase);
  uint32_t cls_mask[4] = {0u, 0u, 0u, 0u};
  uint64_t dtab = 0;                              // d per row, 3 bits each
#pragma unroll
  for (int rr = 0; rr < kR; ++rr) {
    const int tb0 = static_cast<int>((32u - ((e0 + static_cast<uint32_t>(rr) * static_cast<uint32_t>(L)) & 31u)) & 31u);
    const int key = rev ? ((tb0 - 1) & 31) : tb0;
    cls_mask[key >> 3] |= 1u << rr;
    dtab |= static_cast<uint64_t>(key & 7) << (3 * rr);
  }
  // Stores the item [lo, hi) of row rr (lanes 32 h .. 32 h + 31) from the ring.
  auto flush_item = [&](int rr, int lo, int hi) {
    const int t = lo + (lane & 31);
    const int s0 = lo % Lay::RING_T + (lane & 31);
    const int slot = s0 >= Lay::RING_T ? s0 - Lay::RING_T : s0;
    const float vu = ring[rr * Lay::RING_T + slot];
    const float vd = ring[(kR + rr) * Lay::RING_T + slot];
    const uint32_t o = pin_u(t < hi ? (static_cast<uint32_t>(rr) * static_cast<uint32_t>(L) +
                                       static_cast<uint32_t>(t)) * 4u
                                    : kOob);
    bstore<float>(rDu, o, vu);
    bstore<float>(rDd, o, vd);
  };
  auto flush_lines = [&](int j, bool last) {
    const int w = j * T;
    uint32_t m = cls_mask[j & 3];
    while (m != 0) {                              // two rows per pass, 32 lanes each
      int rr[2], lo[2], hi[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rr[h] = m != 0 ? __builtin_ctz(m) : 0;
        const int d = static_cast<int>((dtab >> (3 * rr[h])) & 7u);
        if (rev) {
          hi[h] = w + 1 + d;
          lo[h] = hi[h] - 32 > 0 ? hi[h] - 32 : 0;
          if (m == 0 || hi[h] > L) hi[h] = lo[h];         // (the tail item takes it)
        } else {
          lo[h] = w + d;
          hi[h] = lo[h] + 32 < L ? lo[h] + 32 : L;
          if (m == 0) hi[h] = lo[h];
        }
        m &= m - 1;
      }
      const bool h1 = lane >= 32;
      flush_item(h1 ? rr[1] : rr[0], h1 ? lo[1] : lo[0], h1 ? hi[1] : hi[0]);
    }
    if (last) {                                   // the partial line at the far end of every row
#pragma unroll 1
      for (int rr = 0; rr < kR; rr += 2) {
        int lo2[2], hi2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tb0 = static_cast<int>(
              (32u - ((e0 + static_cast<uint32_t>(rr + h) * static_cast<uint32_t>(L)) & 31u)) & 31u);
          if (rev) {
            const int tl = L - ((L - tb0) & 31);  // last boundary <= L
            lo2[h] = tl > 0 ? tl : 0;
            hi2[h] = L;
          } else {
            lo2[h] = 0;
            hi2[h] = tb0 < L ? tb0 : L;
          }
        }
        const bool h1 = lane >= 32;
        flush_item(rr + (h1 ? 1 : 0), h1 ? lo2[1] : lo2[0], h1 ? hi2[1] : hi2[0]);
      }
    }
  };

  const int n_bc = lane % 16;
  uint32_t bo[BQ];
#pragma unroll
  for (int i = 0; i < BQ; ++i) {
    const int q = lane / 16 + 4 * i;
    const int qt = rev ? T - 1 - q : q;
    bo[i] = n_bc < dstate ? (static_cast<uint32_t>(n_bc) * static_cast<uint32_t>(P.bsn) +
                             static_cast<uint32_t>(qt) * static_cast<uint32_t>(P.bst)) * 4u
                          : kOob;
  }
  const uint32_t bst_bytes = static_cast<uint32_t>(P.bst) * 4u;
  const bool sp_on = p.softplus != 0;

  auto tile_of = [&](int k) { return rev ? nt - 1 - k : k; };
  // Raw global values of the next tile (loaded one tile ahead, so that their
  // latency overlaps the current tile's arithmetic).  Steps past L and rows
  // past dim read 0.
  float lu[PE], ld[PE], ly[PE], lb[BQ], lc[BQ], lk[kNS];
  const uint32_t ck_lane = static_cast<uint32_t>(r * 16 + n0) * 4u;
  const uint32_t dy_tile_bytes = static_cast<uint32_t>(p.dy_tiled ? 16 * T : T) * 4u;
  auto stage_load = [&](int j, bool pass2) {
    const int jT = j * T;
    const bool in_seq = tq < L - jT;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const uint32_t o = pin_u(in_seq ? ob[i] + static_cast<uint32_t>(jT) * 4u : kOob);
      lu[i] = bload<float>(rU, o);
      ld[i] = bload<float>(rDl, o);
      // (tile-major dy has slots for all 16 rows of the block; rows past dim
      // read 0, as they do from the flat layout, whose range ends at dim)
      ly[i] = pass2 ? bload<float>(rDy, pin_u(in_seq && srow[i] < rows
                                                  ? oy[i] + static_cast<uint32_t>(j) * dy_tile_bytes : kOob))
                    : 0.0f;
    }
    const uint32_t tb = static_cast<uint32_t>(jT) * bst_bytes;
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      lb[i] = bload<float>(rB, bo[i] + tb);
      lc[i] = pass2 ? bload<float>(rC, bo[i] + tb) : 0.0f;
    }
    if (pass2) {
      bload4(rCk, ck_lane + static_cast<uint32_t>(j) * 1024u, lk);
    } else {
#pragma unroll
      for (int jn = 0; jn < kNS; ++jn) lk[jn] = 0.0f;
    }
  };
  // Stages the loaded tile: (dt, dt u, dy) per element ((dt, u, dy) with
  // ZOH) and B, C per step into LDS, and keeps the element values the tile's
  // combine needs.
  float eu[PE], edt[PE], edy[PE], ex[PE];
  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const float uv = pin(lu[i]);
      const float x = pin(ld[i]) + sbias[i];
      const float dyv = pin(ly[i]);
      const float dtv = sp_on ? softplus_f(x) : x;
      eu[i] = uv;
      edt[i] = dtv;
      edy[i] = dyv;
      ex[i] = x;
      *reinterpret_cast<float4 *>(prep + srow[i] * Lay::PST + 4 * sq) =
          make_float4(dtv, ZOH ? uv : dtv * uv, dyv, 0.0f);
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      float *const q = bcs + (lane / 16 + 4 * i) * 32 + n_bc;
      q[0] = pin(lb[i]);
      q[16] = pin(lc[i]);
    }
  };

  // ---- pass 1: states at every tile start, in visit order (unless the
  // forward kernel that recomputed the output stored them already)
  float h[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) h[j] = 0.0f;
  const int nt1 = p.ck_ready ? 0 : nt;
  if (nt1 > 0) stage_load(tile_of(0), false);
  for (int k = 0; k < nt1; ++k) {
    const int j = tile_of(k);
    bstore4(rCk, ck_lane + static_cast<uint32_t>(j) * 1024u, h);
    wave_lds_fence();                    // the previous tile's staged values are read
    stage_store();
    wave_lds_fence();
    stage_load(tile_of(k + 1 < nt1 ? k + 1 : nt1 - 1), false);
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const float4 pq = *reinterpret_cast<const float4 *>(prep + r * Lay::PST + 4 * q);
      const float bv = bcs[q * 32 + bc_slot];
#pragma unroll
      for (int jn = 0; jn < kNS; ++jn) {
        const float x2 = pq.x * A2[jn];
        const float a = hw_exp2(x2);
        float w;
        switch (jn) {
          case 0: w = pq.y * row_bcast<0>(bv); break;
          case 1: w = pq.y * row_bcast<1>(bv); break;
          case 2: w = pq.y * row_bcast<2>(bv); break;
          default: w = pq.y * row_bcast<3>(bv); break;
        }
        if constexpr (ZOH) w *= zoh_coef(pq.x, x2, a, iA[jn]);
        h[jn] = __builtin_fmaf(a, h[jn], w);
      }
    }
  }
  // the checkpoints written above are read back below
  __syncthreads();

  // ---- pass 2: tiles in reverse visit order
  float gn[kNS], dA[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    gn[j] = 0.0f;
    dA[j] = 0.0f;
  }
  // Sums over the block's channels per (n, step) of tile j: dC_t of dy_t h_t,
  // dB_t of g_t dt_t u_t.  The contributions meet in LDS, the dB ones in the
  // same area after the dC ones are read (each hand-over between lanes
  // ordered by wave_lds_fence).
  auto reduce_red = [&](const Rsrc &dst, int j) {
#pragma unroll
    for (int m = 0; m < 16 * T / 64; ++m) {
      const int c = lane + 64 * m;                  // (n, q), q fastest
      const int q = c % T, n = c / T;
      const float4 *src = reinterpret_cast<const float4 *>(red + c * Lay::RSTR + (n / 4) * 16);
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < kR / 4; ++v) {
        const float4 x4 = src[v];
        sum += (x4.x + x4.y) + (x4.z + x4.w);
      }
      bstore<float>(dst, static_cast<uint32_t>((j * 16 + n) * T + (rev ? T - 1 - q : q)) * 4u, sum);
    }
  };
  // A tile's last stores (its dB sums and the output lines it completes) go
  // out in the next iteration, before that iteration's loads: vector memory
  // counts loads and stores in one in-order counter, so stores issued after
  // a tile's loads would hold up the wait for those loads.
  auto finish_tile = [&](int j, bool last) {
    if constexpr (!ZOH) flush_lines(j, last);
    reduce_red(rPB, j);
  };
  stage_load(tile_of(nt - 1), true);
  for (int k = nt - 1; k >= 0; --k) {
    const int j = tile_of(k);
    wave_lds_fence();                    // the previous tile's partial sums are read
    stage_store();
    wave_lds_fence();
    float hc[kNS], h0[kNS];
#pragma unroll
    for (int jn = 0; jn < kNS; ++jn) {
      // (channels past dim: a checkpoint written by a forward kernel with
      // the 8-lane split may not cover them; their state stays zero)
      hc[jn] = r < rows ? pin(lk[jn]) : 0.0f;
      h0[jn] = hc[jn];
    }
    if (k < nt - 1) {
      finish_tile(tile_of(k + 1), false);
      wave_lds_fence();                  // its dB sums are read before the dC ones are written
    }
    stage_load(tile_of(k > 0 ? k - 1 : 0), true);
    // recompute the tile's states and decays (the staged step values and
    // B, C stay in registers for the adjoint)
    float hs[T][kNS], as[T][kNS];
    float4 pqs[T];
    float bvs[T];
#pragma unroll
    for (int q = 0; q < T; ++q) {
      pqs[q] = *reinterpret_cast<const float4 *>(prep + r * Lay::PST + 4 * q);
      bvs[q] = bcs[q * 32 + bc_slot];
    }
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const float4 pq = pqs[q];
      const float bv = bvs[q];
#pragma unroll
      for (int jn = 0; jn < kNS; ++jn) {
        const float x2 = pq.x * A2[jn];
        const float a = hw_exp2(x2);
        float w;
        switch (jn) {
          case 0: w = pq.y * row_bcast<0>(bv); break;
          case 1: w = pq.y * row_bcast<1>(bv); break;
          case 2: w = pq.y * row_bcast<2>(bv); break;
          default: w = pq.y * row_bcast<3>(bv); break;
        }
        if constexpr (ZOH) w *= zoh_coef(pq.x, x2, a, iA[jn]);
        hc[jn] = __builtin_fmaf(a, hc[jn], w);
        hs[q][jn] = hc[jn];
        as[q][jn] = a;
      }
    }
    const int jT = j * T;
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
      for (int jn = 0; jn < kNS; ++jn)
        red[((n0 + jn) * T + q) * Lay::RSTR + sp * 16 + r] = pqs[q].z * hs[q][jn];
    wave_lds_fence();
    reduce_red(rPC, j);
    wave_lds_fence();
    // adjoint back through the tile: g = C dy + a_{t+1} g_{t+1} per state
    // (accumulated in place of gn), sum_n g B into sgB, sum_n g a h A into
    // sqA; the B and C broadcasts fold into the multiply-adds
    // (v_fmac_f32_dpp) where the write allows it
#pragma unroll
    for (int q = T - 1; q >= 0; --q) {
      const float4 pq = pqs[q];
      const float bv = bvs[q];
      float sgB = 0.0f, sqA = 0.0f;
#pragma unroll
      for (int jn = 0; jn < kNS; ++jn) {
        float &g = gn[jn];
        switch (jn) {
          case 0: fmac_row_bcast<kNS + 0>(g, bv, pq.z); break;
          case 1: fmac_row_bcast<kNS + 1>(g, bv, pq.z); break;
          case 2: fmac_row_bcast<kNS + 2>(g, bv, pq.z); break;
          default: fmac_row_bcast<kNS + 3>(g, bv, pq.z); break;
        }
        const float ah = as[q][jn] * (q > 0 ? hs[q > 0 ? q - 1 : 0][jn] : h0[jn]);   // a_t h_{t-1}
        const float gq = g * ah;
        if constexpr (ZOH) {
          // pq.y is u; k and dk/dA are recomputed from the kept decay
          float Bb;
          switch (jn) {
            case 0: Bb = row_bcast<0>(bv); break;
            case 1: Bb = row_bcast<1>(bv); break;
            case 2: Bb = row_bcast<2>(bv); break;
            default: Bb = row_bcast<3>(bv); break;
          }
          const float x2 = pq.x * A2[jn];
          const float kq = zoh_coef(pq.x, x2, as[q][jn], iA[jn]);
          const float gBu = g * Bb * pq.y;
          red[((n0 + jn) * T + q) * Lay::RSTR + sp * 16 + r] = g * kq * pq.y;   // dB
          sgB = __builtin_fmaf(g * Bb, kq, sgB);
          dA[jn] = __builtin_fmaf(gq, pq.x, __builtin_fmaf(gBu, zoh_coef_dA(pq.x, x2, as[q][jn], iA[jn], kq),
                                                           dA[jn]));
          sqA = __builtin_fmaf(gq, An[jn], __builtin_fmaf(gBu, as[q][jn], sqA));
        } else {
          switch (jn) {
            case 0: sgB = row_bcast<0>(bv) * g; break;
            case 1: fmac_row_bcast<1>(sgB, bv, g); break;
            case 2: fmac_row_bcast<2>(sgB, bv, g); break;
            default: fmac_row_bcast<3>(sgB, bv, g); break;
          }
          red[((n0 + jn) * T + q) * Lay::RSTR + sp * 16 + r] = g * pq.y;   // dB
          dA[jn] = __builtin_fmaf(gq, pq.x, dA[jn]);
          sqA = __builtin_fmaf(gq, An[jn], sqA);
        }
        g = as[q][jn] * g;
      }
      part[(0 * 64 + lane) * Lay::QSTR + q] = sgB;
      part[(1 * 64 + lane) * Lay::QSTR + q] = sqA;
    }
    // per element: du, ddelta (the four state groups of the channel summed)
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      float gB = 0.0f, gA = 0.0f;
#pragma unroll
      for (int s = 0; s < 64 / kR; ++s) {
        gB += part[(0 * 64 + s * kR + srow[i]) * Lay::QSTR + sq];
        gA += part[(1 * 64 + s * kR + srow[i]) * Lay::QSTR + sq];
      }
      // without ZOH the write's dt u factors out of the state sums
      const float du = ZOH ? __builtin_fmaf(sD[i], edy[i], gB) : __builtin_fmaf(edt[i], gB, sD[i] * edy[i]);
      const float ddt = ZOH ? gA : __builtin_fmaf(eu[i], gB, gA);
      const float sig = hw_rcp(1.0f + hw_exp2(-ex[i] * kLog2e));
      const float dd = sp_on ? ddt * sig : ddt;
      if constexpr (ZOH) {
        const uint32_t o = pin_u(tq < L - jT ? ob[i] + static_cast<uint32_t>(jT) * 4u : kOob);
        bstore<float>(rDu, o, du);
        bstore<float>(rDd, o, dd);
      } else {
        const int slot = (j % (Lay::RING_T / T)) * T + tq;   // t mod RING_T
        ring[srow[i] * Lay::RING_T + slot] = du;
        ring[(kR + srow[i]) * Lay::RING_T + slot] = dd;
      }
      accD[i] = __builtin_fmaf(edy[i], eu[i], accD[i]);
      accB[i] += dd;
    }
  }
  wave_lds_fence();
  finish_tile(tile_of(0), true);

  // ---- per batch row: dA, and dD, dbias (the T lanes of a channel summed)
  const int64_t prow = static_cast<int64_t>(b) * dim + d0;
  const Rsrc rPA = make_rsrc(p.pA + prow * 16, static_cast<uint32_t>(rows) * 64u);
#pragma unroll
  for (int jn = 0; jn < kNS; ++jn)
    bstore<float>(rPA, static_cast<uint32_t>(r * 16 + n0 + jn) * 4u, dA[jn]);
  wave_lds_fence();
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    part[srow[i] * Lay::QSTR + sq] = accD[i];
    part[64 * Lay::QSTR + srow[i] * Lay::QSTR + sq] = accB[i];
  }
  wave_lds_fence();
  if (lane < kR) {
    float sD_ = 0.0f, sB_ = 0.0f;
    for (int q = 0; q < T; ++q) {
      sD_ += part[lane * Lay::QSTR + q];
      sB_ += part[64 * Lay::QSTR + lane * Lay::QSTR + q];
    }
    const Rsrc rPD = make_rsrc(p.pD + prow, static_cast<uint32_t>(rows) * 4u);
    const Rsrc rPb = make_rsrc(p.pbias + prow, static_cast<uint32_t>(rows) * 4u);
    bstore<float>(rPD, static_cast<uint32_t>(lane) * 4u, sD_);
    bstore<float>(rPb, static_cast<uint32_t>(lane) * 4u, sB_);
  }
}

// The reductions of a group's partial sums, all directions in one launch
// (blockIdx.y = direction): blocks below bc_blocks add the dB, dC partials
// over channel blocks, the others (one per channel) the dA, dD, dbias
// partials over batch rows.  Fixed summation orders: deterministic.
struct ReduceJob {
  const float *pB, *pC, *pA, *pD, *pbias;
  float *dB, *dC, *dA, *dD, *dbias;
};
struct ReduceGroup {
  ReduceJob j[kBwdGroupMax];
  int64_t batch, dim, slab;       // slab: floats of one channel block's dB (dC) partials
  int L, dstate, nrb, nt, bc_blocks;
};

// dB, dC [batch, dstate, L] from partials [nrb][batch][tiles][16][T]:
// element e of one block's slab is read in storage order (whole lines) and
// lands at (b, n, t).
__device__ void reduce_bc(const ReduceGroup &g, const ReduceJob &J) {
  constexpr int T = kBwdTile;
  const int64_t per_b = static_cast<int64_t>(g.nt) * 16 * T;
  const int64_t stride = static_cast<int64_t>(g.bc_blocks) * 256;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < g.slab; e += stride) {
    float sb[4] = {0.f, 0.f, 0.f, 0.f}, sc[4] = {0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + 4 <= g.nrb; k += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sb[u] += J.pB[(k + u) * g.slab + e];
        sc[u] += J.pC[(k + u) * g.slab + e];
      }
    }
    for (; k < g.nrb; ++k) {
      sb[0] += J.pB[k * g.slab + e];
      sc[0] += J.pC[k * g.slab + e];
    }
    const int64_t b = e / per_b;
    const int rem = static_cast<int>(e - b * per_b);
    const int j = rem / (16 * T), n = (rem / T) % 16, t = j * T + rem % T;
    if (n < g.dstate && t < g.L) {
      const int64_t o = (b * g.dstate + n) * g.L + t;
      J.dB[o] = (sb[0] + sb[1]) + (sb[2] + sb[3]);
      J.dC[o] = (sc[0] + sc[1]) + (sc[2] + sc[3]);
    }
  }
}

// dA [dim, dstate], dD [dim], dbias [dim] for channel d: thread t adds the
// rows b = t / 16 (mod 16 slices) for state t % 16; the slices meet in LDS.
__device__ void reduce_param(const ReduceGroup &g, const ReduceJob &J, int64_t d) {
  __shared__ float sa[256], sd[256], sb[256];
  const int t = threadIdx.x, n = t & 15, slice = t >> 4;
  float a = 0.f, dd = 0.f, db = 0.f;
  for (int64_t bb = slice; bb < g.batch; bb += 16) {
    a += J.pA[(bb * g.dim + d) * 16 + n];
    if (n == 0) {
      dd += J.pD[bb * g.dim + d];
      db += J.pbias[bb * g.dim + d];
    }
  }
  sa[t] = a;
  sd[t] = dd;
  sb[t] = db;
  __syncthreads();
  if (t < 16) {
    float s = 0.f, s2 = 0.f, s3 = 0.f;
    for (int k = 0; k < 16; ++k) {
      s += sa[k * 16 + t];
      s2 += sd[k * 16 + t];
      s3 += sb[k * 16 + t];
    }
    if (t < g.dstate) J.dA[d * g.dstate + t] = s;
    if (t == 0) {
      J.dD[d] = s2;
      if (J.dbias != nullptr) J.dbias[d] = s3;
    }
  }
}

__global__ void __launch_bounds__(256) reduce_kernel(const ReduceGroup g) {
  const ReduceJob &J = g.j[blockIdx.y];
  if (static_cast<int>(blockIdx.x) < g.bc_blocks) reduce_bc(g, J);
  else reduce_param(g, J, static_cast<int64_t>(blockIdx.x) - g.bc_blocks);
}

// dy = scale * dout * SiLU(z) and dz = scale * dout * y * SiLU'(z), with
// SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z), y = y1 (+ y2 when given);
// without z, dy = scale * dout.
__global__ void __launch_bounds__(256)
gate_bwd_kernel(const float *__restrict__ y, const float *__restrict__ y2, const float *__restrict__ z,
                const float *__restrict__ dout, float *__restrict__ dy, float *__restrict__ dz,
                int64_t n, float scale) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const float g = scale * dout[e];
    if (z == nullptr) {
      dy[e] = g;
    } else {
      const float zv = z[e];
      const float s = hw_rcp(1.0f + hw_exp2(-zv * kLog2e));
      const float yv = y2 != nullptr ? y[e] + y2[e] : y[e];
      dy[e] = g * zv * s;
      dz[e] = g * yv * (s * __builtin_fmaf(zv, 1.0f - s, 1.0f));
    }
  }
}

// out = a + b (+ c when given), elementwise.
__global__ void __launch_bounds__(256)
add_kernel(const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ c,
           float *__restrict__ out, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256)
    out[e] = c != nullptr ? (a[e] + b[e]) + c[e] : a[e] + b[e];
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  const int64_t cap = 256 * 32;
  return static_cast<unsigned>(g < 1 ? 1 : (g < cap ? g : cap));
}

}  // namespace

int64_t scan_bwd_tiles(int64_t L) { return (L + kBwdTile - 1) / kBwdTile; }
int64_t scan_bwd_ck_floats(int64_t batch, int64_t dim, int64_t L) {
  return batch * ((dim + kR - 1) / kR) * scan_bwd_tiles(L) * 256;
}
int64_t scan_bwd_tiled_floats(int64_t batch, int64_t dim, int64_t L) {
  return ((dim + kR - 1) / kR) * batch * scan_bwd_tiles(L) * 16 * kBwdTile;
}

hipError_t launch_scan_bwd_group(const BwdGroup &g, hipStream_t s) {
  if (g.n < 1 || g.n > kBwdGroupMax) return hipErrorInvalidValue;
  const BwdArgs &a = g.a[0];
  for (int k = 1; k < g.n; ++k)
    if (g.a[k].batch != a.batch || g.a[k].dim != a.dim || g.a[k].L != a.L || g.a[k].dstate != a.dstate ||
        g.a[k].zoh != a.zoh || g.a[k].ck_ready != a.ck_ready || g.a[k].dy_tiled != a.dy_tiled)
      return hipErrorInvalidValue;
  const int64_t nrb = (a.dim + kR - 1) / kR;
  const int64_t blocks = a.batch * nrb;
  if (blocks == 0) return hipSuccess;
  const size_t lds = BwdLayout<kBwdTile>::TOTAL * sizeof(float);
  // One direction takes the single-direction kernel; so does each direction
  // of a ZOH group (one wave per SIMD, its registers tight) once one
  // direction has a wave for every SIMD (256 CUs x 4).
  if (g.n == 1 || (a.zoh && blocks >= 1024)) {
    for (int k = 0; k < g.n; ++k) {
      if (a.zoh)
        hipLaunchKernelGGL((scan_bwd_kernel<kBwdTile, true, BwdArgs>), dim3(static_cast<unsigned>(blocks)),
                           dim3(64), lds, s, g.a[k]);
      else
        hipLaunchKernelGGL((scan_bwd_kernel<kBwdTile, false, BwdArgs>), dim3(static_cast<unsigned>(blocks)),
                           dim3(64), lds, s, g.a[k]);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (a.zoh)
    hipLaunchKernelGGL((scan_bwd_kernel<kBwdTile, true, BwdGroup>), dim3(static_cast<unsigned>(blocks * g.n)),
                       dim3(64), lds, s, g);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<kBwdTile, false, BwdGroup>), dim3(static_cast<unsigned>(blocks * g.n)),
                       dim3(64), lds, s, g);
  return hipGetLastError();
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s) {
  BwdGroup g = {};
  g.a[0] = a;
  g.n = 1;
  return launch_scan_bwd_group(g, s);
}

hipError_t launch_scan_bwd_reduce_group(const BwdGroup &g, const BwdReduceOut out[], hipStream_t s) {
  if (g.n < 1 || g.n > kBwdGroupMax) return hipErrorInvalidValue;
  const BwdArgs &a = g.a[0];
  ReduceGroup r = {};
  for (int k = 0; k < g.n; ++k)
    r.j[k] = ReduceJob{g.a[k].pB, g.a[k].pC, g.a[k].pA, g.a[k].pD, g.a[k].pbias,
                       out[k].dB, out[k].dC, out[k].dA, out[k].dD, out[k].dbias};
  r.batch = a.batch;
  r.dim = a.dim;
  r.L = static_cast<int>(a.L);
  r.dstate = a.dstate;
  r.nrb = static_cast<int>((a.dim + kR - 1) / kR);
  r.nt = static_cast<int>(scan_bwd_tiles(a.L));
  r.slab = a.batch * r.nt * 16 * kBwdTile;
  r.bc_blocks = static_cast<int>(grid_for(r.slab));
  hipLaunchKernelGGL(reduce_kernel, dim3(static_cast<unsigned>(r.bc_blocks + a.dim), static_cast<unsigned>(g.n)),
                     dim3(256), 0, s, r);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float *y, const float *z, const float *dout, float *dy, float *dz,
                           int64_t n, float scale, hipStream_t s, const float *y2) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_bwd_kernel, dim3(grid_for(n)), dim3(256), 0, s, y, y2, z, dout, dy, dz, n,
                     scale);
  return hipGetLastError();
}

hipError_t launch_add(const float *a, const float *b, const float *c, float *out, int64_t n,
                      hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3(grid_for(n)), dim3(256), 0, s, a, b, c, out, n);
  return hipGetLastError();
}

}  // namespace vmk
