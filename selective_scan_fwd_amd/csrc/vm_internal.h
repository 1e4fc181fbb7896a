// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <initializer_list>
#include <stdint.h>

namespace vmk {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Rows (channels) per wave and per row block: one lane owns one channel.
constexpr int kRows = 64;

// bf16 values are carried as raw 16-bit patterns.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest, ties to even; NaN stays a (quiet) NaN.
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Hardware 2^x (v_exp_f32) and log2 (v_log_f32), reciprocal (v_rcp_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(e^-|x|).  log1p(e) is taken as
// log(s) - ((s - 1) - e) with s = fl(1 + e): the second term is the rounding
// error of s, which removes it to first order; leaving out its division by s
// changes the result by at most 2^-24 * e / (1 + e), below fp32 resolution of
// log1p(e).  Small e thus keeps full relative accuracy.
// (max(x, 0) is one v_max_f32: written as fmaxf it would first quiet a
// signalling NaN in x with an extra instruction, which a NaN input does not
// need here, since the log term is NaN then too.)
__device__ __forceinline__ float relu_f(float x) {
  float r;
  asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float softplus_f(float x) {
  float e = hw_exp2(-__builtin_fabsf(x) * kLog2e);
  float s = 1.0f + e;
  float corr = (s - 1.0f) - e;
  return relu_f(x) + __builtin_fmaf(hw_log2(s), kLn2, -corr);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X.  Give
// each XCD a contiguous range of logical blocks, so that neighbouring row
// blocks of one batch row (which share B and C) meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  int q = nblocks / kXcd, r = nblocks % kXcd;
  int x = bid % kXcd, k = bid / kXcd;
  return x * q + (x < r ? x : r) + k;
}

// ---------------------------------------------------------------- scan
struct DirPtrs {
  const void *u;        // [batch, dim, L] (Tin)
  const void *delta;    // [batch, dim, L] (Tin)
  const float *A;       // [dim, dstate]
  const void *B;        // element (b, n, t) at b*bsb + n*bsn + t*bst (Tin)
  const void *C;        // same layout as B
  int64_t bsb, bsn, bst;
  const float *D;       // [dim]
  const float *bias;    // [dim] or nullptr
  const float *cw;      // [dim, 4] causal conv weights (conv scans) or nullptr
  const float *cb;      // [dim] conv bias or nullptr
};

struct ScanArgs {
  DirPtrs dir[2];
  const void *z;        // [batch, dim, L] (Tin) or nullptr
  void *out;            // [batch, dim, L] (Tin)
  float *xglobal;       // fp32 exchange rows (long bidirectional), row stride xstride
  int64_t xstride;
  // Backward preparation: per direction, the state at every 8-step tile
  // start (checkpoints laid out as BwdArgs::ck; kOptCk, or kOptBwdPrep when
  // dy is set); with kOptBwdPrep also, in place of out, the gate's backward
  // from the ungated y: dy = gscale dout SiLU(z), tile-major as BwdArgs::dy
  // with dy_tiled, and dz = gscale dout y SiLU'(z) ([batch, dim, L]), both
  // fp32.
  float *ck[2];
  const float *gz, *dout;
  float *dy, *dz;
  float gscale;
  int64_t batch, dim, L;
  int dstate;
  int softplus;
  int zoh;              // zero-order-hold input coefficient instead of dt
  int conv;             // u holds the conv input x; the scan uses SiLU(conv(x))
  int reverse;          // one-direction scans only
  float scale;          // bidirectional combine scale
  int prio_from;        // (set at launch) first workgroup past the first round
};

// Kernel variants (template bits of the scan kernel).  kOptCk stores the
// backward's checkpoints (ck) only; kOptBwdPrep also forms the gate's
// backward in place of out (on-chip exchange).
enum ScanOpt { kOptZoh = 1, kOptConv = 2, kOptBwdPrep = 4, kOptCk = 8 };

// Where a bidirectional scan parks first-visit sums: in LDS (short
// sequences) or in fp32 global memory.
enum XMode { kXNone = 0, kXLds = 1, kXGlobal = 2 };

struct ScanPlan {
  int S;        // lanes sharing one channel's 16 states (state split)
  int T;        // tile length in steps
  int dirs;     // 1 or 2
  int xmode;    // XMode
  int sub;      // row blocks per workgroup
  size_t lds;   // dynamic LDS bytes per workgroup
  int threads;  // workgroup size: 64 dirs sub
  int64_t blocks;
  // Sequence-parallel scan (one direction, few rows): chunks > 1 runs the
  // chunked kernel, one workgroup per channel whose lanes own `chunks`
  // sub-chunks of chunk_len consecutive steps of the visit order.
  int chunks;
  int chunk_len;
};

ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t L, int dstate, int dirs, bool conv);
// Row stride (floats) of the global exchange buffer: rows padded to whole
// 128-byte lines so that no two channels' parked partials share a line.
int64_t xchg_global_stride(int64_t L);
// Whether every in-kernel offset of this launch fits 32 bits.
bool scan_offsets_fit(const ScanPlan &plan, const ScanArgs &args, bool bf16);
hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &args, bool bf16, hipStream_t s);
hipError_t launch_scan_chunked(const ScanPlan &plan, const ScanArgs &args, bool bf16, hipStream_t s);

// ---------------------------------------------------------------- backward
// One direction, fp32.  dy: gradient of the ungated scan output, [batch,
// dim, L], or with dy_tiled [batch][nrb][tiles][16 channels][8 steps] (one
// contiguous 512-byte block per row block and tile; positions past L are
// never read).  The kernel
// writes du and ddelta per element and partial sums that the reduce kernel
// adds: pB, pC [nrb][batch][tiles][16 states][8 steps] (per block of 16
// channels, one contiguous 512-byte block per tile), pA [batch][dim][16],
// pD, pbias [batch][dim].  ck: state checkpoints (scratch),
// [batch][nrb][tiles][16 channels][16 states], so that one wave's
// checkpoints of one tile are one contiguous kilobyte.
struct BwdArgs {
  DirPtrs dir;
  const float *dy;
  float *du, *ddelta;
  float *ck, *pA, *pD, *pbias, *pB, *pC;
  int64_t batch, dim, L;
  int dstate;
  int softplus;
  int zoh;              // zero-order-hold write
  int reverse;
  int ck_ready;         // ck already holds the checkpoints (the forward kernel wrote them)
  int dy_tiled;         // dy is tile-major (the forward kernel wrote it)
};
constexpr int kBwdTile = 8;
int64_t scan_bwd_tiles(int64_t L);
// Floats of the checkpoint buffer, and of a tile-major buffer (pB, pC, a
// tiled dy).
int64_t scan_bwd_ck_floats(int64_t batch, int64_t dim, int64_t L);
int64_t scan_bwd_tiled_floats(int64_t batch, int64_t dim, int64_t L);
hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s);
// Up to four directions' backward kernels in one launch (one grid over all
// of them): the same batch, dim, L and dstate, the same zoh and ck_ready.
constexpr int kBwdGroupMax = 4;
struct BwdGroup {
  BwdArgs a[kBwdGroupMax];
  int n;
};
hipError_t launch_scan_bwd_group(const BwdGroup &g, hipStream_t s);
// The sums of the partials of every direction of a group, in one launch.
struct BwdReduceOut {
  float *dA, *dB, *dC, *dD, *dbias;
};
hipError_t launch_scan_bwd_reduce_group(const BwdGroup &g, const BwdReduceOut out[], hipStream_t s);
// dy = scale dout SiLU(z), dz = scale dout (y + y2) SiLU'(z) (y2 may be null;
// without z, dy = scale dout).
hipError_t launch_gate_bwd(const float *y, const float *z, const float *dout, float *dy, float *dz,
                           int64_t n, float scale, hipStream_t s, const float *y2 = nullptr);
// out = a + b (+ c when not null)
hipError_t launch_add(const float *a, const float *b, const float *c, float *out, int64_t n,
                      hipStream_t s);

// ---------------------------------------------------------------- layout
hipError_t launch_atrous_gather(const void *x, void *streams, int64_t batch, int64_t ch,
                                int64_t H, int64_t W, bool bf16, hipStream_t s);
hipError_t launch_atrous_scatter(const void *streams, void *y, int64_t batch, int64_t ch,
                                 int64_t H, int64_t W, bool bf16, hipStream_t s);
hipError_t launch_mean_pool(const void *u, float *pooled, int64_t rows, int64_t H, int64_t W,
                            int axis, bool bf16, hipStream_t s);
hipError_t launch_repeat_gate(const float *y, const void *z, void *out, int64_t rows, int64_t H,
                              int64_t W, int axis, float scale, bool bf16, hipStream_t s);
// Backward of the repeat + gate (dy [rows][Lp] fp32, dz [rows][H][W] fp32 or
// null without z) and of the mean pool (du [rows][H][W] fp32).
hipError_t launch_repeat_gate_bwd(const float *y, const void *z, const void *dout, float *dy, float *dz,
                                  int64_t rows, int64_t H, int64_t W, int axis, float scale, bool bf16,
                                  hipStream_t s);
hipError_t launch_pool_bwd(const float *dubar, float *du, int64_t rows, int64_t H, int64_t W, int axis,
                           hipStream_t s);
hipError_t launch_to_f32(const void *src, float *dst, int64_t n, hipStream_t s);
// Causal depthwise conv1d (width 4) + SiLU over [rows][L] (row = b * dim + d).
hipError_t launch_conv1d_silu(const void *x, const float *w, const float *cb, void *out,
                              int64_t rows, int64_t L, int64_t dim, int reverse, bool bf16,
                              hipStream_t s);
// Its backward: dx [rows][L] fp32, dw [dim][4], dcb [dim] (or null) fp32 from
// du [rows][L] fp32; partial: conv1d_bwd_chunks(...) * dim * 5 floats.
int conv1d_bwd_chunks(int64_t batch, int64_t dim, int *rows_per_chunk);
hipError_t launch_conv1d_silu_bwd(const void *x, const float *w, const float *cb, const float *du,
                                  float *dx, float *dw, float *dcb, float *partial, int64_t batch,
                                  int64_t dim, int64_t L, int reverse, bool bf16, hipStream_t s);
// [planes][H][W] -> [planes][W][H]
hipError_t launch_transpose(const void *in, void *out, int64_t planes, int64_t H, int64_t W, bool bf16,
                            hipStream_t s);
// out = scale * (yr + transpose(yc)) * SiLU(z); yr [planes][H][W] fp32 (may
// be out), yc [planes][W][H] fp32, z / out in the token dtype.
hipError_t launch_ss2d_merge(const float *yr, const float *yc, const void *z, void *out,
                             int64_t planes, int64_t H, int64_t W, float scale, bool bf16,
                             hipStream_t s);
// The fused four-wide forms of the SS2D backward's layout steps (fp32): they
// need H % 4 == 0, W % 4 == 0 and 16-byte aligned tensors (ss2d_tile4_ok),
// else hipErrorInvalidValue.  Gate backward: y = yr + transpose(yc),
// dy = scale dout SiLU(z) in [planes][H][W] and dyt = its [planes][W][H]
// transpose, dz = scale dout y SiLU'(z); z NULL: dy = scale dout.
bool ss2d_tile4_ok(int64_t H, int64_t W, std::initializer_list<const void *> ptrs);
hipError_t launch_ss2d_gate_bwd(const float *yr, const float *yc, const float *z, const float *dout,
                                float *dy, float *dyt, float *dz, int64_t planes, int64_t H, int64_t W,
                                float scale, hipStream_t s);
// du = (d0 + d1) + transpose(d2 + d3); d0, d1, du [planes][H][W], d2, d3 [planes][W][H].
hipError_t launch_ss2d_du_sum(const float *d0, const float *d1, const float *d2, const float *d3,
                              float *du, int64_t planes, int64_t H, int64_t W, hipStream_t s);

}  // namespace vmk
