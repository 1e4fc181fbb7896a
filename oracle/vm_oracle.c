/*
 * vm_oracle.c -- fp64 CPU oracle for the selective-scan hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it is written directly from the pages'
 * statement of the method, in plain sequential loops, in double precision.
 *
 * Sources (web pages; cited by title and section):
 *  [Vim]  "Vision Mamba: Bidirectional State Space Models for Images"
 *         (abhik.ai): sections "A state retains, writes, and reads",
 *         "Two scans meet at the same token", "Inside the released Vim block",
 *         and implementation rows 4 ("Keep a running state, then read it")
 *         and 5 ("Align the backward scan before combining").
 *  [EVM]  "EfficientVMamba: Atrous Selective Scan for Light Weight Visual
 *         Mamba" (abhik.ai): sections "Four shorter sequences, one dense
 *         output", "Merge restores coordinates instead of adding directions",
 *         "What the selective state carries", implementation rows 1-3.
 *  [FVim] "Fast Vision Mamba: Pooling Spatial Dimensions for Accelerated
 *         Processing" (gptget.net summary): "Methodology" and "Key Findings".
 *  [NoD]  "Norm or Direction? Decoding Vision Mambas for High-Resolution
 *         Vision": section 3 "Background" (eq. 1-2, and "2D Selective Scan
 *         (SS2D)").
 *
 * Readings where the pages leave a step open are listed at each function.
 * Every function returns 0 on success and a negative value on bad arguments.
 * All arrays are dense, row-major (C order), in the shapes documented below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define VMO_EBADARG (-1)
#define VMO_ENOMEM (-2)

int vmo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* softplus(x) = log(1 + e^x), written in the overflow-free form
 * max(x, 0) + log1p(e^{-|x|}), which is the same function.  [Vim] row 3 and
 * row 4 make the step size positive with softplus after adding the bias. */
static double softplus(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* SiLU(z) = z * sigmoid(z): the signed, unbounded gate ([Vim] "Inside the
 * released Vim block"). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Input coefficient of the state write for step size dt and decay a.
 * Released recurrence ([Vim] "A state retains, writes, and reads" and row 4):
 * dt, i.e. the write is dt * B * u.  Exact zero-order hold ([NoD] eq. 2 for a
 * diagonal A; the same passage of [Vim] states the scalar form): with A, B and
 * u held constant over the step, the write is (exp(dt a) - 1) / a * B * u,
 * whose limit at a = 0 is dt * B * u.  expm1 keeps the digits that
 * exp(dt a) - 1 cancels when dt a is small.
 */
static double write_coef(double dt, double a, int zoh) {
  if (!zoh) return dt;
  return a != 0.0 ? expm1(dt * a) / a : dt;
}

/*
 * One channel of one sequence, visited in increasing t from a zero state
 * ([Vim] "A state retains, writes, and reads": each directional scan starts
 * from zero; row 4 equations):
 *
 *   x_t   = delta_t + bias
 *   dt_t  = softplus(x_t)  if delta_softplus, else x_t
 *   h_t,n = exp(dt_t * A_n) * h_{t-1,n} + k(dt_t, A_n) * B_n,t * u_t
 *   y_t   = sum_n C_n,t * h_t,n + D * u_t
 *
 * with k = write_coef (dt_t, or the zero-order-hold coefficient when zoh).
 * u, delta, y: [L] with element stride 1.  A: [N].  B, C: [N][L] (the batch's
 * slice, shared by every channel).  h: scratch of N doubles.
 */
static void scan_channel(const double *u, const double *delta, const double *A,
                         const double *B, const double *C, double D,
                         double bias, int delta_softplus, int zoh, int64_t L,
                         int64_t N, double *h, double *y) {
  for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    double x = delta[t] + bias;
    double dt = delta_softplus ? softplus(x) : x;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double retain = exp(dt * A[n]);
      double write = write_coef(dt, A[n], zoh) * B[n * L + t] * u[t];
      h[n] = retain * h[n] + write;
      acc += C[n * L + t] * h[n];
    }
    y[t] = acc + D * u[t];
  }
}

/* Reverse the order of the last axis of a [rows][L] block into dst. */
static void flip_rows(const double *src, double *dst, int64_t rows, int64_t L) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t t = 0; t < L; ++t) dst[r * L + t] = src[r * L + (L - 1 - t)];
}

/*
 * Selective scan, one direction.
 *   u, delta, z, out: [batch][dim][L]     A: [dim][N]
 *   B, C: [batch][N][L]                   D, delta_bias: [dim]
 * z and delta_bias may be NULL (no gate / zero bias).  With z the output is
 * y * SiLU(z) ([Vim] row 4 returns the gated output when z is given).
 * zoh != 0 selects the zero-order-hold input coefficient (write_coef).
 *
 * reverse != 0 is the backward direction of [Vim] "Two scans meet at the same
 * token" and row 5: the whole sequence (every token tensor, including z) is
 * reversed, scanned forward, and the result is reversed back, so that the
 * output is indexed by original token position.  This is done literally here
 * (flip, scan, flip), not by walking indices backwards.
 */
int vmo_selective_scan(const double *u, const double *delta, const double *A,
                       const double *B, const double *C, const double *D,
                       const double *z, const double *delta_bias,
                       int64_t batch, int64_t dim, int64_t L, int64_t N,
                       int delta_softplus, int zoh, int reverse, double *out) {
  if (!u || !delta || !A || !B || !C || !D || !out) return VMO_EBADARG;
  if (batch <= 0 || dim <= 0 || L <= 0 || N <= 0) return VMO_EBADARG;
  int status = 0;
#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
    double *ybuf = (double *)malloc(sizeof(double) * (size_t)L);
    double *uf = NULL, *df = NULL, *zf = NULL, *Bf = NULL, *Cf = NULL;
    int64_t flipped_batch = -1;
    if (reverse) {
      uf = (double *)malloc(sizeof(double) * (size_t)L);
      df = (double *)malloc(sizeof(double) * (size_t)L);
      zf = (double *)malloc(sizeof(double) * (size_t)L);
      Bf = (double *)malloc(sizeof(double) * (size_t)(N * L));
      Cf = (double *)malloc(sizeof(double) * (size_t)(N * L));
    }
    int ok = h && ybuf && (!reverse || (uf && df && zf && Bf && Cf));
    if (!ok) {
#pragma omp atomic write
      status = VMO_ENOMEM;
    }
#pragma omp for schedule(static)
    for (int64_t row = 0; row < batch * dim; ++row) {
      if (!ok) continue;
      int64_t b = row / dim, d = row % dim;
      const double *ur = u + row * L, *dr = delta + row * L;
      const double *zr = z ? z + row * L : NULL;
      const double *Bb = B + b * N * L, *Cb = C + b * N * L;
      double bias = delta_bias ? delta_bias[d] : 0.0;
      if (!reverse) {
        scan_channel(ur, dr, A + d * N, Bb, Cb, D[d], bias, delta_softplus, zoh,
                     L, N, h, ybuf);
        for (int64_t t = 0; t < L; ++t)
          out[row * L + t] = zr ? ybuf[t] * silu(zr[t]) : ybuf[t];
      } else {
        if (flipped_batch != b) {
          flip_rows(Bb, Bf, N, L);
          flip_rows(Cb, Cf, N, L);
          flipped_batch = b;
        }
        flip_rows(ur, uf, 1, L);
        flip_rows(dr, df, 1, L);
        if (zr) flip_rows(zr, zf, 1, L);
        scan_channel(uf, df, A + d * N, Bf, Cf, D[d], bias, delta_softplus, zoh,
                     L, N, h, ybuf);
        if (zr)
          for (int64_t t = 0; t < L; ++t) ybuf[t] *= silu(zf[t]);
        flip_rows(ybuf, out + row * L, 1, L);
      }
    }
    free(h); free(ybuf); free(uf); free(df); free(zf); free(Bf); free(Cf);
  }
  return status;
}

/*
 * Depthwise causal convolution of kernel width 4 with bias, then SiLU, on
 * each channel's token sequence ([Vim] "Inside the released Vim block": the
 * content of each branch passes through its own depthwise kernel-four causal
 * Conv1d, then SiLU; the substitution list of the Vim page's reference code
 * states it as a grouped conv1d with left padding, then SiLU):
 *
 *   v_t = bias + sum_{k=0..3} w[k] * x_{t-3+k}   (x_s = 0 for s < 0)
 *   out_t = SiLU(v_t)
 *
 * so w[3] weights the current token and w[0] the token three steps back.
 * reverse != 0 is the backward branch, which reverses the sequence before its
 * convolution: here literally flip, convolve causally, flip back, so the
 * output is in original token order.
 *   x, out: [batch][dim][L]     w: [dim][4]     bias: [dim] (NULL = 0)
 */
int vmo_causal_conv1d_silu(const double *x, const double *w, const double *bias,
                           int64_t batch, int64_t dim, int64_t L, int reverse,
                           double *out) {
  if (!x || !w || !out || batch <= 0 || dim <= 0 || L <= 0) return VMO_EBADARG;
  double *src = (double *)malloc(sizeof(double) * (size_t)L);
  double *dst = (double *)malloc(sizeof(double) * (size_t)L);
  if (!src || !dst) { free(src); free(dst); return VMO_ENOMEM; }
  for (int64_t row = 0; row < batch * dim; ++row) {
    const int64_t d = row % dim;
    if (reverse) flip_rows(x + row * L, src, 1, L);
    else memcpy(src, x + row * L, sizeof(double) * (size_t)L);
    for (int64_t t = 0; t < L; ++t) {
      double v = bias ? bias[d] : 0.0;
      for (int k = 0; k < 4; ++k) {
        const int64_t s = t - 3 + k;
        if (s >= 0) v += w[d * 4 + k] * src[s];
      }
      dst[t] = silu(v);
    }
    if (reverse) flip_rows(dst, out + row * L, 1, L);
    else memcpy(out + row * L, dst, sizeof(double) * (size_t)L);
  }
  free(src); free(dst);
  return 0;
}

/*
 * Bidirectional combine ([Vim] "Two scans meet at the same token", row 5,
 * and "Inside the released Vim block"):
 *   out = scale * (Y_fwd + flip(Y_bwd_on_flipped_input)) * SiLU(z)
 * The backward direction has its own u, delta, A, B, C, D and bias, given in
 * original token order; its scan runs on the reversed sequence and its output
 * is reversed back before the sum (vmo_selective_scan with reverse = 1).
 * scale = 1/2 is the released averaging model, scale = 1 the summed form of
 * the paper's algorithm.  The gate is applied once, after the sum (the page
 * notes this equals gating each direction before the sum).  z may be NULL.
 */
int vmo_bidir_scan(const double *uf, const double *df, const double *Af,
                   const double *Bf, const double *Cf, const double *Df,
                   const double *biasf, const double *ub, const double *db,
                   const double *Ab, const double *Bb, const double *Cb,
                   const double *Db, const double *biasb, const double *z,
                   double scale, int64_t batch, int64_t dim, int64_t L,
                   int64_t N, int delta_softplus, int zoh, double *out) {
  if (!out || batch <= 0 || dim <= 0 || L <= 0) return VMO_EBADARG;
  size_t total = (size_t)(batch * dim * L);
  double *yf = (double *)malloc(sizeof(double) * total);
  double *yb = (double *)malloc(sizeof(double) * total);
  if (!yf || !yb) { free(yf); free(yb); return VMO_ENOMEM; }
  int s = vmo_selective_scan(uf, df, Af, Bf, Cf, Df, NULL, biasf, batch, dim, L,
                             N, delta_softplus, zoh, 0, yf);
  if (s == 0)
    s = vmo_selective_scan(ub, db, Ab, Bb, Cb, Db, NULL, biasb, batch, dim, L,
                           N, delta_softplus, zoh, 1, yb);
  if (s == 0)
    for (size_t i = 0; i < total; ++i) {
      double y = (yf[i] + yb[i]) * scale;
      out[i] = z ? y * silu(z[i]) : y;
    }
  free(yf); free(yb);
  return s;
}

/*
 * p = 2 atrous routes ([EVM] "Four shorter sequences, one dense output" and
 * row 1).  Group k has offset (row, col) = (0,0), (1,0), (0,1), (1,1) for
 * k = 0..3.  Groups 0 and 2 walk the half-resolution grid row-major, groups 1
 * and 3 column-major; no group is reversed.  The grid is padded on the right
 * and bottom to even size, so every group has ceil(H/2) * ceil(W/2) steps.
 * Writes the visited (row, col) of step t of group k into rows[t], cols[t];
 * coordinates with row >= H or col >= W are padding.
 */
int64_t vmo_atrous_group_len(int64_t H, int64_t W) {
  if (H <= 0 || W <= 0) return VMO_EBADARG;
  return ((H + 1) / 2) * ((W + 1) / 2);
}

int vmo_atrous_route(int64_t H, int64_t W, int group, int64_t *rows,
                     int64_t *cols) {
  static const int off_row[4] = {0, 1, 0, 1};
  static const int off_col[4] = {0, 0, 1, 1};
  if (H <= 0 || W <= 0 || group < 0 || group > 3 || !rows || !cols)
    return VMO_EBADARG;
  int64_t hr = (H + 1) / 2, hc = (W + 1) / 2, t = 0;
  if (group % 2 == 0) {
    for (int64_t r = 0; r < hr; ++r)
      for (int64_t c = 0; c < hc; ++c, ++t) {
        rows[t] = 2 * r + off_row[group];
        cols[t] = 2 * c + off_col[group];
      }
  } else {
    for (int64_t c = 0; c < hc; ++c)
      for (int64_t r = 0; r < hr; ++r, ++t) {
        rows[t] = 2 * r + off_row[group];
        cols[t] = 2 * c + off_col[group];
      }
  }
  return 0;
}

/*
 * Gather ([EVM] row 1): x [batch][ch][H][W] -> streams [batch][4][ch][Lg];
 * step t of group k holds x at the route's coordinate, or +0.0 where the
 * coordinate is padding.
 */
int vmo_atrous_gather(const double *x, int64_t batch, int64_t ch, int64_t H,
                      int64_t W, double *streams) {
  int64_t Lg = vmo_atrous_group_len(H, W);
  if (!x || !streams || batch <= 0 || ch <= 0 || Lg <= 0) return VMO_EBADARG;
  int64_t *rr = (int64_t *)malloc(sizeof(int64_t) * (size_t)Lg);
  int64_t *cc = (int64_t *)malloc(sizeof(int64_t) * (size_t)Lg);
  if (!rr || !cc) { free(rr); free(cc); return VMO_ENOMEM; }
  for (int k = 0; k < 4; ++k) {
    vmo_atrous_route(H, W, k, rr, cc);
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t c = 0; c < ch; ++c) {
        const double *plane = x + (b * ch + c) * H * W;
        double *s = streams + ((b * 4 + k) * ch + c) * Lg;
        for (int64_t t = 0; t < Lg; ++t)
          s[t] = (rr[t] < H && cc[t] < W) ? plane[rr[t] * W + cc[t]] : 0.0;
      }
  }
  free(rr); free(cc);
  return 0;
}

/*
 * Scatter / merge ([EVM] "Merge restores coordinates ..." and row 3): each
 * valid coordinate takes the value of the single step that visited it; padded
 * steps are dropped (crop).  Nothing is summed.  streams [batch][4][ch][Lg]
 * -> y [batch][ch][H][W].
 */
int vmo_atrous_scatter(const double *streams, int64_t batch, int64_t ch,
                       int64_t H, int64_t W, double *y) {
  int64_t Lg = vmo_atrous_group_len(H, W);
  if (!streams || !y || batch <= 0 || ch <= 0 || Lg <= 0) return VMO_EBADARG;
  int64_t *rr = (int64_t *)malloc(sizeof(int64_t) * (size_t)Lg);
  int64_t *cc = (int64_t *)malloc(sizeof(int64_t) * (size_t)Lg);
  if (!rr || !cc) { free(rr); free(cc); return VMO_ENOMEM; }
  for (int k = 0; k < 4; ++k) {
    vmo_atrous_route(H, W, k, rr, cc);
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t c = 0; c < ch; ++c) {
        double *plane = y + (b * ch + c) * H * W;
        const double *s = streams + ((b * 4 + k) * ch + c) * Lg;
        for (int64_t t = 0; t < Lg; ++t)
          if (rr[t] < H && cc[t] < W) plane[rr[t] * W + cc[t]] = s[t];
      }
  }
  free(rr); free(cc);
  return 0;
}

/*
 * Mean over one spatial axis ([FVim] "Methodology": parameter-free mean
 * pooling of the (h, w) grid after the convolution).
 *   u [batch][dim][H][W] -> pooled [batch][dim][Lp]
 *   axis 0: mean over W (one value per grid row, Lp = H)
 *   axis 1: mean over H (one value per grid column, Lp = W)
 * The sum runs in index order and is divided by the pooled extent.
 */
int vmo_mean_pool(const double *u, int64_t batch, int64_t dim, int64_t H,
                  int64_t W, int axis, double *pooled) {
  if (!u || !pooled || batch <= 0 || dim <= 0 || H <= 0 || W <= 0 ||
      (axis != 0 && axis != 1))
    return VMO_EBADARG;
  for (int64_t r = 0; r < batch * dim; ++r) {
    const double *g = u + r * H * W;
    if (axis == 0) {
      for (int64_t i = 0; i < H; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < W; ++j) s += g[i * W + j];
        pooled[r * H + i] = s / (double)W;
      }
    } else {
      for (int64_t j = 0; j < W; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < H; ++i) s += g[i * W + j];
        pooled[r * W + j] = s / (double)H;
      }
    }
  }
  return 0;
}

/*
 * FastVim pooled scan ([FVim] "Methodology"): pool u along one axis, run the
 * forward (and, if given, backward) selective scan on the pooled sequence
 * with the pooled-token delta, B and C, repeat the scan output along the
 * pooled axis back to the full grid, and gate with SiLU of the full-resolution
 * z.  The D skip belongs to the scan and therefore acts on the pooled input.
 *   uf, ub, z, out: [batch][dim][H][W]      df, db: [batch][dim][Lp]
 *   Bf, Cf, Bb, Cb: [batch][N][Lp]           Af, Ab: [dim][N]
 *   out[b,d,i,j] = scale * (yf + yb)[b,d,p] * SiLU(z[b,d,i,j]),
 *   p = i (axis 0) or j (axis 1).  ub == NULL selects forward only
 *   (out = scale * yf * gate).  z == NULL means no gate.
 */
int vmo_pool_scan_repeat(const double *uf, const double *df, const double *Af,
                         const double *Bf, const double *Cf, const double *Df,
                         const double *biasf, const double *ub,
                         const double *db, const double *Ab, const double *Bb,
                         const double *Cb, const double *Db,
                         const double *biasb, const double *z, double scale,
                         int64_t batch, int64_t dim, int64_t H, int64_t W,
                         int64_t N, int axis, int delta_softplus, int zoh,
                         double *out) {
  if (!uf || !out || batch <= 0 || dim <= 0 || H <= 0 || W <= 0 ||
      (axis != 0 && axis != 1))
    return VMO_EBADARG;
  int64_t Lp = axis == 0 ? H : W;
  size_t pn = (size_t)(batch * dim * Lp);
  double *pf = (double *)malloc(sizeof(double) * pn);
  double *pb = (double *)malloc(sizeof(double) * pn);
  double *yf = (double *)malloc(sizeof(double) * pn);
  double *yb = (double *)malloc(sizeof(double) * pn);
  int s = (pf && pb && yf && yb) ? 0 : VMO_ENOMEM;
  if (s == 0) s = vmo_mean_pool(uf, batch, dim, H, W, axis, pf);
  if (s == 0)
    s = vmo_selective_scan(pf, df, Af, Bf, Cf, Df, NULL, biasf, batch, dim, Lp,
                           N, delta_softplus, zoh, 0, yf);
  if (s == 0 && ub) {
    s = vmo_mean_pool(ub, batch, dim, H, W, axis, pb);
    if (s == 0)
      s = vmo_selective_scan(pb, db, Ab, Bb, Cb, Db, NULL, biasb, batch, dim,
                             Lp, N, delta_softplus, zoh, 1, yb);
  }
  if (s == 0) {
    for (int64_t r = 0; r < batch * dim; ++r)
      for (int64_t i = 0; i < H; ++i)
        for (int64_t j = 0; j < W; ++j) {
          int64_t p = axis == 0 ? i : j;
          double y = yf[r * Lp + p] + (ub ? yb[r * Lp + p] : 0.0);
          y *= scale;
          int64_t e = (r * H + i) * W + j;
          out[e] = z ? y * silu(z[e]) : y;
        }
  }
  free(pf); free(pb); free(yf); free(yb);
  return s;
}

/*
 * Four-direction 2-D selective scan with aligned summation ("Norm or
 * Direction? Decoding Vision Mambas for High-Resolution Vision", section 3
 * "Background", paragraph "2D Selective Scan (SS2D)": the feature map is
 * traversed top-to-bottom, bottom-to-top, left-to-right and right-to-left,
 * each sequence goes through its own S6 scan and the outputs are put back
 * in the 2-D layout; [EVM] "Merge restores coordinates instead of adding
 * directions": in dense SS2D every pixel receives an output from every
 * direction and the aligned outputs are summed).
 *
 * Direction k = 0 visits the H x W grid row-major (step t at pixel
 * (t / W, t % W)), k = 1 the same order reversed, k = 2 column-major (step t
 * at pixel (t % H, t / H)), k = 3 that order reversed.  u is the one map
 * [batch][dim][H][W] all four traverse.  Direction k's delta_k, B_k, C_k are
 * indexed by the step of its base order (row-major for k = 0, 1,
 * column-major for k = 2, 3), like the two directions of vmo_bidir_scan;
 * each direction has its own A, D and bias.
 *
 * Here each traversal is written out as a list of pixel positions, u is
 * gathered along it, scanned with vmo_selective_scan (reverse = 1 for the
 * reversed orders) and the result is added back at the same positions:
 *   out = scale * (sum_k y_k) * SiLU(z)      (z may be NULL)
 */
int vmo_ss2d_scan(const double *u, const double *const delta[4],
                  const double *const A[4], const double *const B[4],
                  const double *const C[4], const double *const D[4],
                  const double *const bias[4], const double *z, double scale,
                  int64_t batch, int64_t dim, int64_t H, int64_t W, int64_t N,
                  int delta_softplus, int zoh, double *out) {
  if (!u || !out || batch <= 0 || dim <= 0 || H <= 0 || W <= 0 || N <= 0)
    return VMO_EBADARG;
  for (int k = 0; k < 4; ++k)
    if (!delta[k] || !A[k] || !B[k] || !C[k] || !D[k]) return VMO_EBADARG;
  const int64_t L = H * W, rows = batch * dim;
  int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
  double *uk = (double *)malloc(sizeof(double) * (size_t)(rows * L));
  double *yk = (double *)malloc(sizeof(double) * (size_t)(rows * L));
  int s = (pos && uk && yk) ? 0 : VMO_ENOMEM;
  for (int64_t e = 0; s == 0 && e < rows * L; ++e) out[e] = 0.0;
  for (int k = 0; s == 0 && k < 4; ++k) {
    for (int64_t t = 0; t < L; ++t)   /* pixel (i, j) as flat i * W + j */
      pos[t] = k < 2 ? t : (t % H) * W + t / H;
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t t = 0; t < L; ++t) uk[r * L + t] = u[r * L + pos[t]];
    s = vmo_selective_scan(uk, delta[k], A[k], B[k], C[k], D[k], NULL, bias[k],
                           batch, dim, L, N, delta_softplus, zoh, k % 2, yk);
    for (int64_t r = 0; s == 0 && r < rows; ++r)
      for (int64_t t = 0; t < L; ++t) out[r * L + pos[t]] += yk[r * L + t];
  }
  for (int64_t e = 0; s == 0 && e < rows * L; ++e) {
    double y = scale * out[e];
    out[e] = z ? y * silu(z[e]) : y;
  }
  free(pos); free(uk); free(yk);
  return s;
}
