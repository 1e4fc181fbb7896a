/*
 * vm_scan.h -- C ABI of the selective-scan hot path for vision Mamba
 * backbones (Vim bidirectional blocks, EfficientVMamba atrous ES2D, FastVim
 * pooled scan, four-direction SS2D) on AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are dense, contiguous, row-major, in the shapes given at each
 *    call, and live in device memory of the current HIP device.  The caller
 *    owns every buffer; the library never frees or keeps a pointer past the
 *    call.  Outputs must not overlap any input (checked: VM_ERR_ALIAS).
 *  - dtype selects the storage of the token tensors (u, delta, z, B, C, x,
 *    streams, out): VM_F32 or VM_BF16.  A, D and delta_bias are always fp32.
 *    Arithmetic is fp32 (bf16 inputs are widened exactly; bf16 outputs are
 *    rounded to nearest even).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Argument checks run on the host first and nothing is
 *    launched when they fail.  Kernel-side faults surface at the caller's next
 *    synchronisation; VM_ERR_HIP reports a launch failure.
 *  - No data-dependent checks run on the device: A <= 0, finite inputs and a
 *    non-negative step size are preconditions of the method, and NaN / Inf
 *    propagate by IEEE rules.
 *  - Some calls need temporary device memory (noted at the call); it comes
 *    from a stream-ordered pool owned by the library and is released on the
 *    same stream before the call returns (VM_ERR_ALLOC if unavailable).
 *  - Calls are thread-safe.
 *
 * The pages this follows (cited by title and section):
 *  [Vim]  "Vision Mamba: Bidirectional State Space Models for Images"
 *  [EVM]  "EfficientVMamba: Atrous Selective Scan for Light Weight Visual Mamba"
 *  [FVim] "Fast Vision Mamba: Pooling Spatial Dimensions for Accelerated
 *         Processing"
 *  [NoD]  "Norm or Direction? Decoding Vision Mambas for High-Resolution
 *         Vision"
 */
#ifndef VM_SCAN_H
#define VM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of token tensors. */
enum { VM_F32 = 0, VM_BF16 = 1 };

/* Status codes returned by every entry point. */
enum {
  VM_OK = 0,
  VM_ERR_NULL = 1,        /* a required pointer is NULL                      */
  VM_ERR_SHAPE = 2,       /* a size is <= 0, or an element count overflows   */
  VM_ERR_DTYPE = 3,       /* unknown dtype                                    */
  VM_ERR_FLAG = 4,        /* a flag or pool_axis is not 0/1, or options has
                             unknown bits                                     */
  VM_ERR_ALIAS = 5,       /* the output overlaps an input                     */
  VM_ERR_UNSUPPORTED = 6, /* dstate outside [1, 16], a non-finite scale, or
                             sizes past the kernels' 32-bit offsets or grid
                             limits: 32 rows of seqlen + 16 steps, or one
                             batch row of B or C, must span < 2 GiB; the map
                             calls (atrous, pooled, SS2D) take at most
                             2^24 - 1 planes (batch * channels), the scans
                             at most 2^24 - 1 row blocks of 16 channels
                             (batch * ceil(dim / 16))                         */
  VM_ERR_HIP = 7,         /* a HIP launch or runtime call failed              */
  VM_ERR_ALLOC = 8        /* temporary device memory could not be obtained    */
};

/*
 * Options of the scan entry points (`options`, bitwise OR; any other bit is
 * VM_ERR_FLAG):
 *   VM_DELTA_SOFTPLUS  dt = softplus(delta + bias); without it dt = delta + bias
 *   VM_ZOH             write with the exact zero-order-hold coefficient
 *                      (exp(dt A) - 1) / A in place of dt ([NoD] section 3,
 *                      eq. 2, for diagonal A; [Vim] "A state retains, writes,
 *                      and reads" gives the scalar form and notes that the
 *                      released recurrence uses dt).  Its A -> 0 limit is dt.
 *                      Evaluated in fp32 to within about 5e-7 relative,
 *                      including small dt A, where exp(dt A) - 1 would cancel.
 * The released Vim model is options = VM_DELTA_SOFTPLUS.
 */
enum { VM_DELTA_SOFTPLUS = 1, VM_ZOH = 2 };

/* Human-readable name of a status code (static storage; never NULL). */
const char *vm_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int vm_version(void);

/*
 * One scan direction, in the argument order of the selective-scan function
 * on [Vim] implementation row 4 ("Keep a running state, then read it"):
 *   u           [batch, dim, seqlen]    token content (dtype)
 *   delta       [batch, dim, seqlen]    step-size pre-activation (dtype),
 *                                       before bias and softplus
 *   A           [dim, dstate]  fp32     decay; A = -exp(A_log), so A <= 0
 *   B, C        [batch, dstate, seqlen] input write / output read (dtype),
 *                                       shared by all channels of a batch row
 *   D           [dim]          fp32     direct skip (required)
 *   delta_bias  [dim]          fp32     added to delta before softplus; NULL = 0
 *   bc_stride   storage of B and C:
 *                 0   dense [batch, dstate, seqlen] as written above;
 *                 >0  token-major: element (b, n, t) at (b*seqlen + t)*bc_stride
 *                     + n, i.e. the [batch, dstate, seqlen] tensors are
 *                     transposed views of [batch, seqlen, >= dstate] memory.
 *                     This is how the page's projection produces B and C (it
 *                     splits the projected tokens and passes transposed
 *                     views); both layouts are read in place.
 *                     Requires bc_stride >= dstate.
 *   conv_w      [dim, 4]       fp32     NULL: u is the scan input as given.
 *                                       Non-NULL: u holds the content x before
 *                                       the block's depthwise causal conv, and
 *                                       the scan input is computed on the fly
 *                                       as SiLU(conv(x)) (vm_causal_conv1d_silu,
 *                                       with this direction's reverse sense);
 *                                       the D skip uses that input.  Only
 *                                       vm_selective_scan_fwd and
 *                                       vm_bidir_scan_fwd (both directions or
 *                                       neither) accept it; elsewhere
 *                                       VM_ERR_UNSUPPORTED.
 *   conv_b      [dim]          fp32     conv bias; NULL = 0 (ignored without
 *                                       conv_w)
 * For vm_pool_scan_repeat the shapes differ (see there).
 */
typedef struct vm_scan_dir {
  const void *u;
  const void *delta;
  const float *A;
  const void *B;
  const void *C;
  const float *D;
  const float *delta_bias;
  int64_t bc_stride;
  const float *conv_w;
  const float *conv_b;
} vm_scan_dir;

/*
 * Selective scan, one direction ([Vim] "A state retains, writes, and reads"
 * and implementation row 4).  For every (b, d), from a zero state:
 *   dt_t   = softplus(delta_t + bias_d)   (options & VM_DELTA_SOFTPLUS)
 *          = delta_t + bias_d             (otherwise)
 *   h_t,n  = exp(dt_t A_d,n) h_t-1,n + k_t,n B_b,n,t u_t
 *   k_t,n  = dt_t, or (exp(dt_t A_d,n) - 1) / A_d,n with VM_ZOH
 *   y_t    = sum_n C_b,n,t h_t,n + D_d u_t
 *   out_t  = y_t * SiLU(z_t)   (z != NULL),   y_t otherwise
 * reverse = 1 visits t = seqlen-1 .. 0 instead, which equals reversing every
 * token tensor, scanning forward and reversing the result ([Vim] "Two scans
 * meet at the same token").  All tensors stay in original token order.
 *   z, out: [batch, dim, seqlen] (dtype).  dstate in [1, 16].
 */
int vm_selective_scan_fwd(const vm_scan_dir *p, const void *z, void *out,
                          int64_t batch, int64_t dim, int64_t seqlen,
                          int64_t dstate, int dtype, int options,
                          int reverse, void *stream);

/*
 * Bidirectional scan with the aligned combine and shared gate ([Vim] "Two
 * scans meet at the same token", "Inside the released Vim block",
 * implementation row 5):
 *   out = combine_scale * (y_fwd + y_bwd) * SiLU(z)
 * y_fwd is the forward scan of `fwd`; y_bwd is the reversed-order scan of
 * `bwd` (its own u, delta, A, B, C, D, bias), returned in original order.
 * combine_scale = 0.5 is the released averaging model, 1 the summed form.
 * z may be NULL (no gate).  out: [batch, dim, seqlen] (dtype).
 * Temporary memory: for sequences too long for the on-chip exchange buffer
 * (seqlen above 552; 520 with a fused conv), an fp32 [batch, dim, seqlen rounded up to 32]
 * exchange buffer from the library's stream-ordered pool.  With VM_F32, a
 * seqlen that is a multiple of 32 and a 128-byte aligned `out`, `out` itself
 * serves as the exchange buffer and nothing is allocated.
 */
int vm_bidir_scan_fwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd,
                      const void *z, float combine_scale, void *out,
                      int64_t batch, int64_t dim, int64_t seqlen,
                      int64_t dstate, int dtype, int options,
                      void *stream);

/*
 * vm_bidir_scan_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and checks as vm_bidir_scan_fwd, and
 * the same kernels; it calls no hipMalloc, hipFree or allocating routine.
 * Where vm_bidir_scan_fwd would take its exchange buffer from the pool (a
 * sequence past the on-chip exchange whose `out` cannot serve), this entry
 * uses a library-owned device array of 8 Mi fp32 values (32 MiB; one per
 * GPU the library runs on, held until the process ends):
 *   batch * dim * (seqlen rounded up to 32) must be at most 8388608, else
 *   VM_ERR_UNSUPPORTED (checked on the host before any HIP call).
 * Every call on one GPU shares that array and leaves its contents behind
 * (each exchange row is written before it is read, so nothing needs
 * clearing): calls that overlap in time on one GPU (different streams or
 * host threads) race and must not be issued.
 */
int vm_bidir_scan_fwd_noalloc(const vm_scan_dir *fwd, const vm_scan_dir *bwd,
                              const void *z, float combine_scale, void *out,
                              int64_t batch, int64_t dim, int64_t seqlen,
                              int64_t dstate, int dtype, int options,
                              void *stream);

/*
 * Depthwise causal convolution of width 4 with bias, then SiLU: the step
 * that produces the scan input u from the block's content x ([Vim] "Inside
 * the released Vim block": each branch's content passes through its own
 * kernel-four causal Conv1d, then SiLU; the backward branch reverses the
 * sequence first).  For every row (b, d):
 *   forward      u_t = SiLU(bias_d + sum_k w_d,k x_{t-3+k})
 *   reverse = 1  u_t = SiLU(bias_d + sum_k w_d,k x_{t+3-k})
 * with x = 0 outside [0, seqlen): w_d,3 weights the current token, w_d,0 the
 * token three steps earlier in the direction's visit order, and the
 * convolution does not reach across rows.
 *   x, out [batch, dim, seqlen] (dtype); w [dim, 4] fp32; bias [dim] fp32
 *   (NULL = 0).  The same result feeds the block's projections of delta, B
 *   and C; the scan entry points can recompute it from x (conv_w).
 * Limit: batch * dim * seqlen below 2^33 elements (VM_ERR_UNSUPPORTED).
 */
int vm_causal_conv1d_silu(const void *x, const float *w, const float *bias,
                          void *out, int64_t batch, int64_t dim,
                          int64_t seqlen, int reverse, int dtype,
                          void *stream);

/*
 * Backward of vm_causal_conv1d_silu: the gradients of L = sum(du * u) for
 * the same x, w, bias and direction (the pages pin gradients only as
 * automatic differentiation of the forward loop).  With dv = du SiLU'(v),
 * v the convolution plus bias:
 *   dx_t  = sum_k w_d,k dv_{t+3-k}  (forward; reverse: dv_{t-3+k})
 *   dw_d,k = sum over b, t of dv_t x_{t-3+k}  (reverse: x_{t+3-k})
 *   dbias_d = sum over b, t of dv_t
 *   x [batch, dim, seqlen] (dtype); w [dim, 4], bias [dim] (NULL = 0) fp32;
 *   du [batch, dim, seqlen] fp32 (the scan backward's u gradient);
 *   dx [batch, dim, seqlen], dw [dim, 4] fp32; dbias [dim] fp32 or NULL
 *   (not computed).  Outputs must not overlap the inputs or each other
 *   (VM_ERR_ALIAS).  dw and dbias are summed in a fixed order
 *   (deterministic).
 * Temporary memory: per-chunk partial sums, about 2048 * 5 floats.
 * Limits: dim at most 2^24 - 1, and seqlen times the rows of one chunk below
 * 2^31 (VM_ERR_UNSUPPORTED).
 */
int vm_causal_conv1d_silu_bwd(const void *x, const float *w, const float *bias,
                              const float *du, float *dx, float *dw, float *dbias,
                              int64_t batch, int64_t dim, int64_t seqlen, int reverse,
                              int dtype, void *stream);

/*
 * Number of steps of each p = 2 atrous group: ceil(H/2) * ceil(W/2)
 * ([EVM] implementation row 1).  Returns -VM_ERR_SHAPE for H or W <= 0.
 * Pure host function.
 */
int64_t vm_atrous_group_len(int64_t height, int64_t width);

/*
 * Atrous gather, p = 2 ([EVM] "Four shorter sequences, one dense output",
 * implementation row 1).  x [batch, channels, H, W] -> streams
 * [batch, 4, channels, Lg].  Group k has offset (row, col) = (0,0), (1,0),
 * (0,1), (1,1); groups 0 and 2 walk the half grid row-major, 1 and 3
 * column-major.  The map is padded right/bottom to even size; padded steps
 * hold +0.0.  A bit-exact copy.
 */
int vm_atrous_gather(const void *x, void *streams, int64_t batch,
                     int64_t channels, int64_t height, int64_t width,
                     int dtype, void *stream);

/*
 * Atrous scatter / merge ([EVM] "Merge restores coordinates instead of adding
 * directions", implementation row 3): the inverse routing, then a crop of the
 * padding.  streams [batch, 4, channels, Lg] -> y [batch, channels, H, W];
 * each valid coordinate takes its single owner's value; nothing is summed.
 * A bit-exact copy.
 */
int vm_atrous_scatter(const void *streams, void *y, int64_t batch,
                      int64_t channels, int64_t height, int64_t width,
                      int dtype, void *stream);

/*
 * FastVim pooled scan ([FVim] "Methodology"): mean-pool u over one spatial
 * axis, run the selective scan on the pooled tokens (forward, plus backward
 * when bwd != NULL), repeat the result along the pooled axis, gate with the
 * full-resolution SiLU(z):
 *   out[b,d,i,j] = combine_scale * (y_fwd + y_bwd)[b,d,p] * SiLU(z[b,d,i,j])
 *   p = i, Lp = H for pool_axis = 0 (mean over W)
 *   p = j, Lp = W for pool_axis = 1 (mean over H)
 * Per direction: u [batch, dim, H, W] (full resolution), delta [batch, dim,
 * Lp], B and C [batch, dstate, Lp] (the pooled tokens' projections), A, D,
 * delta_bias as for vm_selective_scan_fwd.  The D skip acts on the pooled u.
 * z, out: [batch, dim, H, W].  z may be NULL.  Temporary memory: fp32
 * [batch, dim, Lp] buffers for the pooled u of each direction and the scan
 * result, and fp32 copies of delta, B and C with VM_BF16.
 */
int vm_pool_scan_repeat(const vm_scan_dir *fwd, const vm_scan_dir *bwd,
                        const void *z, float combine_scale, void *out,
                        int64_t batch, int64_t dim, int64_t height,
                        int64_t width, int64_t dstate, int pool_axis,
                        int dtype, int options, void *stream);

/*
 * Four-direction 2-D selective scan with summed merge ([NoD] section 3,
 * "2D Selective Scan (SS2D)": four traversals of the map, one S6 scan each,
 * outputs restored to the map and merged; the merge of full SS2D adds the
 * four aligned outputs, [EVM] "Merge restores coordinates instead of adding
 * directions"):
 *   traversal 0: row-major, pixel (i, j) at step i*W + j
 *   traversal 1: traversal 0 reversed
 *   traversal 2: column-major, pixel (i, j) at step j*H + i
 *   traversal 3: traversal 2 reversed
 *   out[b,d,i,j] = combine_scale * sum_k y_k[b,d,(i,j)] * SiLU(z[b,d,i,j])
 * u, z, out: [batch, dim, H, W] (dtype); z may be NULL.  dirs[4]: the four
 * traversals' parameters; dirs[k].u is ignored (every traversal reads u).
 * delta [batch, dim, H*W] and B, C [batch, dstate, H*W] (or token-major, see
 * bc_stride) are indexed by traversal step: row-major for traversals 0 and 1,
 * column-major for 2 and 3.  A traversal's D skip adds D * u at each pixel,
 * so the merged skip is (D_0 + D_1 + D_2 + D_3) * u.  The H and W 32-pixel
 * tile counts multiplied must not exceed 65535 (VM_ERR_UNSUPPORTED).
 * Temporary memory: fp32 [batch, dim, H, W] buffers for the transposed u and
 * the column traversals' sum, plus (VM_BF16) the row traversals' sum and fp32
 * copies of u, delta, B and C, plus the exchange buffers of long sequences as
 * in vm_bidir_scan_fwd.
 */
int vm_ss2d_scan_fwd(const vm_scan_dir *dirs, const void *u, const void *z,
                     float combine_scale, void *out, int64_t batch,
                     int64_t dim, int64_t height, int64_t width,
                     int64_t dstate, int dtype, int options,
                     void *stream);

/*
 * Gradients of one scan direction (fp32 device buffers, owned by the
 * caller).  dB and dC are dense [batch, dstate, seqlen] whatever the layout
 * of B and C; ddelta_bias may be NULL (not computed).
 */
typedef struct vm_scan_grad {
  float *du;           /* [batch, dim, seqlen] */
  float *ddelta;       /* [batch, dim, seqlen] */
  float *dA;           /* [dim, dstate]        */
  float *dB;           /* [batch, dstate, seqlen] */
  float *dC;           /* [batch, dstate, seqlen] */
  float *dD;           /* [dim]                */
  float *ddelta_bias;  /* [dim] or NULL        */
  /* With the fused conv (conv_w in the direction, whose u is then the conv
     input x): du receives the gradient with respect to x, and these the
     conv parameters' (dconv_b NULL = not computed).  Unused otherwise. */
  float *dconv_w;      /* [dim, 4]             */
  float *dconv_b;      /* [dim] or NULL        */
} vm_scan_grad;

/*
 * Backward pass of vm_selective_scan_fwd: the gradients of
 * L = sum(dout * out) with respect to every input, for the same arguments
 * (the pages pin the backward pass only as automatic differentiation of the
 * scan loop, [Vim] "A state retains, writes, and reads" and implementation
 * row 4; the adjoint recurrence it implies is g_t = C_t dy_t + a_{t+1} g_{t+1}).
 *   dout [batch, dim, seqlen] (dtype); g: the gradients (see vm_scan_grad);
 *   dz [batch, dim, seqlen] fp32: required exactly when z is given.
 * Gradients are fp32 for either dtype (VM_BF16 inputs are widened exactly
 * and the pass runs in fp32).  Either write (options as the forward call's:
 * with VM_ZOH the derivatives of k = expm1(dt A) / A are included, A = 0
 * among them), with or without the fused conv (see vm_scan_grad).  Gradient buffers must not
 * overlap any input or each other (VM_ERR_ALIAS).  Sums over batch rows (dA,
 * dD, ddelta_bias) and over channels (dB, dC) are formed from per-block
 * partials in a fixed order, so results are deterministic.
 * Temporary memory: state checkpoints ([batch * dim, seqlen / 8, 16] fp32),
 * the partials ([dim / 16, batch, dstate, seqlen] fp32 for each of dB, dC),
 * with z the recomputed forward output and dy, with VM_BF16 fp32 copies of
 * the token tensors, and with the fused conv the conv output, its gradient
 * and the conv backward's partial sums.
 */
int vm_selective_scan_bwd(const vm_scan_dir *p, const void *z,
                          const void *dout, const vm_scan_grad *g, void *dz,
                          int64_t batch, int64_t dim, int64_t seqlen,
                          int64_t dstate, int dtype, int options, int reverse,
                          void *stream);

/*
 * Backward pass of vm_bidir_scan_fwd: gf and gb receive the gradients of the
 * forward and backward directions' inputs, dz (required when z is given) the
 * gate's.  The same limits and temporary memory as vm_selective_scan_bwd,
 * with checkpoints for each direction and, without VM_ZOH, partials for
 * each direction (both directions' backward kernels run as one launch),
 * plus, with z and sequences too long for the on-chip exchange, the
 * recomputation's fp32 exchange rows (as vm_bidir_scan_fwd).  All temporary
 * memory is taken before the first launch.
 */
int vm_bidir_scan_bwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd,
                      const void *z, const void *dout, float combine_scale,
                      const vm_scan_grad *gf, const vm_scan_grad *gb, void *dz,
                      int64_t batch, int64_t dim, int64_t seqlen,
                      int64_t dstate, int dtype, int options, void *stream);

/*
 * Backward pass of vm_pool_scan_repeat ([FVim] "Methodology"), with the same
 * arguments and dout [batch, dim, H, W] (dtype).  gf (and gb when bwd is
 * given) receive their direction's gradients: du at full resolution
 * [batch, dim, H, W] (the mean pool's backward spreads each pooled
 * gradient times 1/w over its line), the others at the pooled length Lp as
 * in vm_selective_scan_bwd; dz [batch, dim, H, W] fp32, required exactly
 * when z is given.  The pooled output's gradient sums the gated dout over
 * the repeated axis in index order (deterministic).  The same options,
 * limits and temporary memory as the scan backward (at length Lp), plus
 * pooled buffers; no fused conv (VM_ERR_UNSUPPORTED).
 */
int vm_pool_scan_repeat_bwd(const vm_scan_dir *fwd, const vm_scan_dir *bwd,
                            const void *z, const void *dout, float combine_scale,
                            const vm_scan_grad *gf, const vm_scan_grad *gb, void *dz,
                            int64_t batch, int64_t dim, int64_t height, int64_t width,
                            int64_t dstate, int pool_axis, int dtype, int options,
                            void *stream);

/*
 * Backward pass of vm_ss2d_scan_fwd ([NoD] section 3, "2D Selective Scan
 * (SS2D)"), with the same arguments and dout [batch, dim, H, W] (dtype).
 *   grads: four gradient sets, one per traversal, for its delta, A, B, C, D
 *   and delta_bias (their du field is ignored); du [batch, dim, H, W] fp32
 *   receives the map's gradient, summed over the four traversals; dz
 *   [batch, dim, H, W] fp32, required exactly when z is given.
 * The same options and limits as the scan backward at length H * W, and
 * as vm_ss2d_scan_fwd.  Temporary memory: the transposed map, with z the
 * recomputed row and column sums, the output gradient in both layouts,
 * four map gradients, and the scan backward's checkpoints and partials for
 * each traversal (the four backward kernels run as one launch).
 */
int vm_ss2d_scan_bwd(const vm_scan_dir *dirs, const void *u, const void *z,
                     const void *dout, float combine_scale, const vm_scan_grad *grads,
                     float *du, void *dz, int64_t batch, int64_t dim, int64_t height,
                     int64_t width, int64_t dstate, int dtype, int options, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VM_SCAN_H */
