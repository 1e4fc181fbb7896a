// Index-exact data movement around the scan:
//  * p = 2 atrous gather / scatter (EfficientVMamba page, "Four shorter
//    sequences, one dense output" and "Merge restores coordinates instead of
//    adding directions"),
//  * mean pooling over one grid axis and the repeat + SiLU gate back to the
//    full grid (FastVim summary, "Methodology"),
//  * the transposes around the column traversals of the four-direction 2-D
//    scan and its summed merge ("Norm or Direction?" page, section 3,
//    "2D Selective Scan (SS2D)"),
//  * the depthwise width-4 causal convolution + SiLU that produces the scan
//    input u (Vision Mamba page, "Inside the released Vim block"),
//  * bf16 -> fp32 widening of side tensors.
// All of these are HBM-bound streaming kernels: every element is read once
// and written once with coalesced accesses.
#include <initializer_list>

#include "vm_internal.h"

namespace vmk {
namespace {

constexpr int kThreads = 256;
constexpr int kPlaneLds = 16384;  // floats of a staged H x W plane (64 KB)

typedef float vf4_t __attribute__((ext_vector_type(4)));
typedef uint32_t vu2_t __attribute__((ext_vector_type(2)));

// Four consecutive values of T moved as one access: 16 bytes of fp32, or 8
// of bf16.  Streaming (nontemporal) forms serve data touched once.
template <typename T> struct Raw4;
template <> struct Raw4<float> {
  using V = vf4_t;
  static __device__ __forceinline__ V pack(float a, float b, float c, float d) { return V{a, b, c, d}; }
};
template <> struct Raw4<bf16_t> {
  using V = vu2_t;
  static __device__ __forceinline__ V pack(bf16_t a, bf16_t b, bf16_t c, bf16_t d) {
    return V{a | (static_cast<uint32_t>(b) << 16), c | (static_cast<uint32_t>(d) << 16)};
  }
};
template <typename T>
__device__ __forceinline__ typename Raw4<T>::V load_raw4_stream(const T *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Raw4<T>::V *>(p));
}
template <typename T>
__device__ __forceinline__ void store_raw4(T *p, typename Raw4<T>::V v) {
  *reinterpret_cast<typename Raw4<T>::V *>(p) = v;
}
template <typename T>
__device__ __forceinline__ void store_raw4_stream(T *p, typename Raw4<T>::V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<typename Raw4<T>::V *>(p));
}

// Step t of group k -> (row, col) on the padded grid.  Offsets (0,0), (1,0),
// (0,1), (1,1); even groups walk the half grid row-major, odd ones
// column-major.  Position t = a * n + b of a walk with n entries per line
// is tracked incrementally: a thread's next element is kThreads further,
// i.e. (a, b) += (kThreads / n, kThreads % n) with one carry, so no element
// pays an integer division.
struct Walk {
  int a, b, da, db, n;
  __device__ void init(int t, int n_) {
    n = n_;
    a = t / n;
    b = t - a * n;
    da = kThreads / n;
    db = kThreads - da * n;
  }
  __device__ void next() {
    a += da;
    b += db;
    if (b >= n) { b -= n; ++a; }
  }
};

// n consecutive values from global memory into LDS, U loads in flight per
// thread before the first LDS store.
template <typename T>
__device__ __forceinline__ void copy_to_lds(T *dst, const T *__restrict__ src, int n) {
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += U * kThreads) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      v[u] = i < n ? src[i] : T(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

// The same for n a multiple of 4, src and dst aligned to 4 values: one
// streaming load of 4 values per access (the source is read once).
template <typename T>
__device__ __forceinline__ void copy_to_lds4(T *dst, const T *__restrict__ src, int n) {
  using V = typename Raw4<T>::V;
  constexpr int U = 4;
  const int n4 = n / 4;
  for (int i0 = threadIdx.x; i0 < n4; i0 += U * kThreads) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      v[u] = i < n4 ? load_raw4_stream(src + 4 * i) : V{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i < n4) reinterpret_cast<V *>(dst)[i] = v[u];
    }
  }
}

// Rows whose length or start is not a multiple of 4 (the 57 x 57 map: 3249
// pixels per plane, 841 steps per stream), in a tensor whose start is
// aligned to 4 values.  The n values at element offset `base` go to LDS with
// aligned 4-value loads: LDS element (base % 4) + e holds value e.  A chunk
// may cover up to 3 values of the neighbouring rows (read, never used); the
// tensor's last partial chunk is read value by value.  Returns base % 4.
template <typename T>
__device__ __forceinline__ int copy_to_lds_chunks(T *lds, const T *__restrict__ tensor, int64_t base, int n,
                                                  int64_t total) {
  using V = typename Raw4<T>::V;
  constexpr int U = 4;
  const int off = static_cast<int>(base & 3);
  const T *a0 = tensor + (base - off);
  const int n4 = (off + n + 3) / 4;
  const int64_t inside = (total - (base - off)) / 4;    // chunks wholly inside the tensor
  for (int i0 = threadIdx.x; i0 < n4; i0 += U * kThreads) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      v[u] = i < n4 && i < inside ? load_raw4_stream(a0 + 4 * i) : V{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      if (i >= n4) continue;
      if (i < inside) {
        reinterpret_cast<V *>(lds)[i] = v[u];
      } else {
        for (int w = 0; w < 4; ++w)
          lds[4 * i + w] = base - off + 4 * i + w < total ? a0[4 * i + w] : T(0);
      }
    }
  }
  return off;
}

// Writes the n values of a row at element offset `base` of a tensor aligned
// to 4 values: the values before the first 4-value boundary and after the
// last one one by one, the rest as aligned 4-value stores.  f4(t, v) gives
// values t .. t+3 (the last ones may lie past the row: unused).
template <typename T, typename F4>
__device__ __forceinline__ void store_row_chunks(T *tensor, int64_t base, int n, F4 &&f4, bool stream) {
  using V = typename Raw4<T>::V;
  const int lead = static_cast<int>((4 - (base & 3)) & 3);
  const int head = lead < n ? lead : n;
  const int n4 = (n - head) / 4;
  const int tail = n - head - 4 * n4;
  T *row = tensor + base;
  for (int j = threadIdx.x; j < n4; j += kThreads) {
    const int t = head + 4 * j;
    T v[4];
    f4(t, v);
    const V w = Raw4<T>::pack(v[0], v[1], v[2], v[3]);
    if (stream) store_raw4_stream(row + t, w);
    else store_raw4(row + t, w);
  }
  const int e = static_cast<int>(threadIdx.x);
  if (e < head + tail) {
    const int t = e < head ? e : head + 4 * n4 + (e - head);
    T v[4];
    f4(t, v);
    row[t] = v[0];
  }
}

// One workgroup per (b, c) plane: stage the plane in LDS with coalesced
// loads, then emit the four streams with coalesced stores.  Vector path
// (staged, H W and Lg multiples of 4, aligned pointers): 4-value loads and
// stores, each thread emitting 4 consecutive steps of a group.
template <typename T>
__global__ void __launch_bounds__(kThreads)
atrous_gather_kernel(const T *__restrict__ x, T *__restrict__ streams, int64_t ch, int H, int W,
                     int staged, int vec) {
  extern __shared__ unsigned char plane_raw[];
  T *plane = reinterpret_cast<T *>(plane_raw);  // H * W values when staged
  const int64_t pid = blockIdx.x;               // b * ch + c
  const int64_t b = pid / ch, c = pid - b * ch;
  const int hr = (H + 1) / 2, hc = (W + 1) / 2, Lg = hr * hc;
  const T *src = x + pid * H * W;
  if (vec == 2) {
    // rows of any length: aligned 4-value chunks (copy_to_lds_chunks,
    // store_row_chunks); every value computed as on the other paths
    const int off = copy_to_lds_chunks(plane, x, pid * H * W, H * W, gridDim.x * static_cast<int64_t>(H) * W);
    __syncthreads();
    const T *pl = plane + off;
    for (int k = 0; k < 4; ++k) {
      const int n = (k & 1) == 0 ? hc : hr;
      store_row_chunks(streams, ((b * 4 + k) * ch + c) * Lg, Lg,
                       [&](int t, T (&v)[4]) __attribute__((always_inline)) {
        int la = t / n, lb = t - la * n;               // (line, position) of step t
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = (k & 1) == 0 ? la : lb, cc = (k & 1) == 0 ? lb : la;
          const int yy = 2 * r + (k & 1), xx = 2 * cc + (k >> 1);
          v[u] = (yy < H && xx < W) ? pl[yy * W + xx] : T(0);
          if (++lb == n) { lb = 0; ++la; }
        }
      }, false);
    }
    return;
  }
  if (vec) {
    copy_to_lds4(plane, src, H * W);
    __syncthreads();
    for (int k = 0; k < 4; ++k) {
      T *dst = streams + ((b * 4 + k) * ch + c) * Lg;
      const int n = (k & 1) == 0 ? hc : hr;
      for (int e = threadIdx.x; e < Lg / 4; e += kThreads) {
        int la = (4 * e) / n, lb = 4 * e - la * n;  // (line, position) of step 4 e
        T v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = (k & 1) == 0 ? la : lb, cc = (k & 1) == 0 ? lb : la;
          const int yy = 2 * r + (k & 1), xx = 2 * cc + (k >> 1);
          v[u] = (yy < H && xx < W) ? plane[yy * W + xx] : T(0);
          if (++lb == n) { lb = 0; ++la; }
        }
        store_raw4(dst + 4 * e, Raw4<T>::pack(v[0], v[1], v[2], v[3]));
      }
    }
    return;
  }
  if (staged) {
    copy_to_lds(plane, src, H * W);
    __syncthreads();
  }
  for (int k = 0; k < 4; ++k) {
    T *dst = streams + ((b * 4 + k) * ch + c) * Lg;
    Walk w;
    w.init(threadIdx.x, (k & 1) == 0 ? hc : hr);   // (r, c) or (c, r)
    for (int t = threadIdx.x; t < Lg; t += kThreads, w.next()) {
      const int r = (k & 1) == 0 ? w.a : w.b, cc = (k & 1) == 0 ? w.b : w.a;
      const int yy = 2 * r + (k & 1), xx = 2 * cc + (k >> 1);
      T v = T(0);
      if (yy < H && xx < W) v = staged ? plane[yy * W + xx] : src[yy * W + xx];
      dst[t] = v;
    }
  }
}

// Inverse routing ("EfficientVMamba: Atrous Selective Scan for Light Weight
// Visual Mamba", "Merge restores coordinates instead of adding directions"):
// p = 2 routing is a permutation of the padded grid, so scatter inverts it
// and crops.  Pixel (row, col) of the map comes from group
// k = (row & 1) + 2 (col & 1) at that group's step t; each output is copied
// and written once (no sums).  When the plane's four streams fit in LDS they are
// staged there first with coalesced loads; the plane is then written with
// coalesced stores.  Vector path (staged, Lg and W multiples of 4, aligned
// pointers): 4-value streaming loads and stores, each thread writing 4
// consecutive pixels of a row.
template <typename T>
__global__ void __launch_bounds__(kThreads)
atrous_scatter_kernel(const T *__restrict__ streams, T *__restrict__ y, int64_t ch, int H, int W,
                      int staged, int vec) {
  extern __shared__ unsigned char st_raw[];
  T *st = reinterpret_cast<T *>(st_raw);        // [4][Lg] when staged
  const int64_t pid = blockIdx.x;
  const int64_t b = pid / ch, c = pid - b * ch;
  const int hr = (H + 1) / 2, hc = (W + 1) / 2, Lg = hr * hc;
  if (vec == 2) {
    // rows of any length (see the gather): each stream at its own LDS slot
    // of SL values, shifted by its start's offset within a 4-value chunk
    const int SL = (Lg + 3) / 4 * 4 + 4;
    const int64_t total = static_cast<int64_t>(gridDim.x) * 4 * Lg;
    // the four streams' shifts, two bits each (arithmetic, not a table)
    int offs = 0;
    for (int k = 0; k < 4; ++k)
      offs |= copy_to_lds_chunks(st + k * SL, streams, ((b * 4 + k) * ch + c) * Lg, Lg, total) << (2 * k);
    __syncthreads();
    store_row_chunks(y, pid * H * W, H * W, [&](int i, T (&v)[4]) __attribute__((always_inline)) {
      int yy = i / W, xx = i - yy * W;                 // pixel i; then along the row
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = (yy & 1) + 2 * (xx & 1);
        const int sk = k * SL + ((offs >> (2 * k)) & 3);
        const int r = yy >> 1, cc = xx >> 1;
        v[u] = (yy < H) ? st[sk + ((yy & 1) == 0 ? r * hc + cc : cc * hr + r)] : T(0);
        if (++xx == W) { xx = 0; ++yy; }
      }
    }, true);
    return;
  }
  if (vec) {
    for (int k = 0; k < 4; ++k) copy_to_lds4(st + k * Lg, streams + ((b * 4 + k) * ch + c) * Lg, Lg);
    __syncthreads();
    T *dst = y + pid * H * W;
    for (int e = threadIdx.x; e < H * W / 4; e += kThreads) {
      const int yy = (4 * e) / W, x0 = 4 * e - yy * W;
      T v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int xx = x0 + u;
        const int k = (yy & 1) + 2 * (xx & 1);
        const int r = yy >> 1, cc = xx >> 1;
        v[u] = st[k * Lg + ((k & 1) == 0 ? r * hc + cc : cc * hr + r)];
      }
      store_raw4_stream(dst + 4 * e, Raw4<T>::pack(v[0], v[1], v[2], v[3]));
    }
    return;
  }
  if (staged) {
    for (int k = 0; k < 4; ++k) copy_to_lds(st + k * Lg, streams + ((b * 4 + k) * ch + c) * Lg, Lg);
    __syncthreads();
  }
  T *dst = y + pid * H * W;
  Walk w;
  w.init(threadIdx.x, W);                       // (row, col) of the plane
  for (int i = threadIdx.x; i < H * W; i += kThreads, w.next()) {
    const int yy = w.a, xx = w.b;
    const int k = (yy & 1) + 2 * (xx & 1);
    const int r = yy >> 1, cc = xx >> 1;
    const int t = (k & 1) == 0 ? r * hc + cc : cc * hr + r;
    dst[i] = staged ? st[k * Lg + t] : streams[((b * 4 + k) * ch + c) * Lg + t];
  }
}

// Four consecutive values as fp32 (one 16-byte or 8-byte load).
__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const bf16_t *p) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
__device__ __forceinline__ void store4(bf16_t *p, float4 v) {
  const uint32_t a = from_f32<bf16_t>(v.x) | (static_cast<uint32_t>(from_f32<bf16_t>(v.y)) << 16);
  const uint32_t b = from_f32<bf16_t>(v.z) | (static_cast<uint32_t>(from_f32<bf16_t>(v.w)) << 16);
  *reinterpret_cast<uint2 *>(p) = make_uint2(a, b);
}

// Streaming forms (nontemporal hint) for the full-resolution tensors of the
// pooled path, each touched once: measured 5 % faster there.  The SS2D and
// conv kernels keep plain accesses, whose outputs the next kernel reads.
__device__ __forceinline__ float4 load4_stream(const float *p) {
  const vf4_t v = __builtin_nontemporal_load(reinterpret_cast<const vf4_t *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4_stream(const bf16_t *p) {
  const vu2_t v = __builtin_nontemporal_load(reinterpret_cast<const vu2_t *>(p));
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ void store4_stream(float *p, float4 v) {
  const vf4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<vf4_t *>(p));
}
__device__ __forceinline__ void store4_stream(bf16_t *p, float4 v) {
  const vu2_t w = {from_f32<bf16_t>(v.x) | (static_cast<uint32_t>(from_f32<bf16_t>(v.y)) << 16),
                   from_f32<bf16_t>(v.z) | (static_cast<uint32_t>(from_f32<bf16_t>(v.w)) << 16)};
  __builtin_nontemporal_store(w, reinterpret_cast<vu2_t *>(p));
}

// Mean over one axis of each H x W grid: one workgroup per grid (b, d),
// sum times fl(1 / extent).
//  * Vector path (W % 4 == 0, aligned): each thread reads four consecutive
//    values at a time; kThreads/(W/4) grid rows are read per pass, U passes
//    in flight.  axis 0 (mean over W): the W/4 threads of a grid row reduce
//    their partial sums across lanes.  axis 1 (mean over H): the row groups'
//    column partials meet in LDS and are added in group order.
//  * Scalar path otherwise.
template <typename T>
__global__ void __launch_bounds__(kThreads)
mean_pool_kernel(const T *__restrict__ u, float *__restrict__ pooled, int H, int W, int axis,
                 float inv, int vec) {
  __shared__ float part[kThreads * 4];
  const int64_t r = blockIdx.x;
  const T *g = u + r * static_cast<int64_t>(H) * W;
  const int tid = threadIdx.x;
  if (vec) {
    const int q = W / 4;                        // threads per grid row (power of two, <= 64)
    const int rows_per_pass = kThreads / q;
    const int rr = tid / q, cq = tid - rr * q;
    constexpr int U = 4;
    if (axis == 0) {
      float *dst = pooled + r * H;
      for (int i0 = 0; i0 < H; i0 += U * rows_per_pass) {
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {           // loads of U grid rows in flight
          const int i = i0 + u * rows_per_pass + rr;
          s[u] = 0.0f;
          if (i < H) {
            const float4 v = load4_stream(g + static_cast<int64_t>(i) * W + 4 * cq);
            s[u] = (v.x + v.y) + (v.z + v.w);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * rows_per_pass + rr;
          for (int off = q / 2; off > 0; off >>= 1) s[u] += __shfl_xor(s[u], off, q);
          if (cq == 0 && i < H) dst[i] = s[u] * inv;
        }
      }
    } else {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
      for (int i = rr; i < H; i += rows_per_pass) {
        const float4 v = load4_stream(g + static_cast<int64_t>(i) * W + 4 * cq);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      reinterpret_cast<float4 *>(part)[tid] = acc;
      __syncthreads();
      float *dst = pooled + r * W;
      for (int j = tid; j < W; j += kThreads) {
        float s = 0.0f;
        for (int k = 0; k < rows_per_pass; ++k) s += part[(k * q + j / 4) * 4 + (j & 3)];
        dst[j] = s * inv;
      }
    }
    return;
  }
  if (axis == 0) {
    float *dst = pooled + r * H;
    const int wave = tid >> 6, lane = tid & 63;
    for (int i = wave; i < H; i += kThreads / 64) {
      float s = 0.0f;
      for (int j = lane; j < W; j += 64) s += to_f32(g[static_cast<int64_t>(i) * W + j]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) dst[i] = s * inv;
    }
  } else {
    float *dst = pooled + r * W;
    for (int j = tid; j < W; j += kThreads) {
      float s = 0.0f;
      for (int i = 0; i < H; ++i) s += to_f32(g[static_cast<int64_t>(i) * W + j]);
      dst[j] = s * inv;
    }
  }
}

// out[r, i, j] = scale * y[r, p] * SiLU(z[r, i, j]),  p = i (axis 0) or j.
// One workgroup per grid (row r).  Vector path (W % 4 == 0, aligned): four
// consecutive elements per thread and U of them in flight; otherwise the
// threads walk the flat grid tracking (i, j) incrementally.
template <typename T>
__global__ void __launch_bounds__(kThreads)
repeat_gate_kernel(const float *__restrict__ y, const T *__restrict__ z, T *__restrict__ out,
                   int H, int W, int axis, float scale, int vec) {
  const int64_t r = blockIdx.x;
  const int hw = H * W;
  const int Lp = axis == 0 ? H : W;
  const float *yr = y + r * Lp;
  const T *zr = z != nullptr ? z + r * static_cast<int64_t>(hw) : nullptr;
  T *outr = out + r * static_cast<int64_t>(hw);
  if (vec) {
    constexpr int U = 4;
    const int n4 = hw / 4;
    for (int e0 = threadIdx.x; e0 < n4; e0 += U * kThreads) {
      float4 zv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * kThreads;
        zv[u] = (zr != nullptr && e < n4) ? load4_stream(zr + 4 * e) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * kThreads;
        if (e >= n4) break;
        const int i = (4 * e) / W, j = 4 * e - i * W;
        float4 v;
        if (axis == 0) {
          const float a = scale * yr[i];
          v = make_float4(a, a, a, a);
        } else {
          const float4 a = *reinterpret_cast<const float4 *>(yr + j);
          v = make_float4(scale * a.x, scale * a.y, scale * a.z, scale * a.w);
        }
        if (zr != nullptr) {
          v.x *= silu_f(zv[u].x); v.y *= silu_f(zv[u].y);
          v.z *= silu_f(zv[u].z); v.w *= silu_f(zv[u].w);
        }
        store4_stream(outr + 4 * e, v);
      }
    }
    return;
  }
  int i = threadIdx.x / W, j = threadIdx.x - (threadIdx.x / W) * W;
  for (int e = threadIdx.x; e < hw; e += kThreads) {
    float v = scale * yr[axis == 0 ? i : j];
    if (zr != nullptr) v *= silu_f(to_f32(zr[e]));
    outr[e] = from_f32<T>(v);
    j += kThreads;
    while (j >= W) { j -= W; ++i; }
  }
}

// ---- four-direction 2-D scan: the column traversals run on the transposed
// map, and their outputs meet the row traversals' outputs transposed back.
// Both passes move 32 x 32 tiles through LDS so that reads and writes are
// coalesced on either side.
constexpr int kTile = 32;

// out[p][j][i] = in[p][i][j] for a [P][H][W] stack of maps.
template <typename T>
__global__ void __launch_bounds__(kThreads)
transpose_kernel(const T *__restrict__ in, T *__restrict__ out, int H, int W, int tiles_w) {
  __shared__ T tile[kTile][kTile + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;   // 32 x 8 threads
  const T *src = in + pl * H * W;
  T *dst = out + pl * H * W;
  for (int r = ty; r < kTile; r += kThreads / kTile) {
    const int i = i0 + r, j = j0 + tx;
    if (i < H && j < W) tile[r][tx] = src[static_cast<int64_t>(i) * W + j];
  }
  __syncthreads();
  for (int r = ty; r < kTile; r += kThreads / kTile) {
    const int j = j0 + r, i = i0 + tx;
    if (i < H && j < W) dst[static_cast<int64_t>(j) * H + i] = tile[tx][r];
  }
}

// Four-wide forms of the two kernels above for H % 4 == 0, W % 4 == 0 and
// 16-byte aligned planes: 64 x 64 tiles, each thread moving four rows of four
// consecutive values (16 values per thread and array in flight).
constexpr int kTile4 = 64;

template <typename T>
__global__ void __launch_bounds__(kThreads)
transpose4_kernel(const T *__restrict__ in, T *__restrict__ out, int H, int W, int tiles_w) {
  __shared__ float tile[kTile4][kTile4 + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile4, j0 = tj * kTile4;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;   // 16 x 16 threads
  const T *src = in + pl * H * W;
  T *dst = out + pl * H * W;
  float4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = i0 + ty + 16 * k, j = j0 + 4 * tx;
    v[k] = (i < H && j < W) ? load4(src + static_cast<int64_t>(i) * W + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float *t = &tile[ty + 16 * k][4 * tx];
    t[0] = v[k].x; t[1] = v[k].y; t[2] = v[k].z; t[3] = v[k].w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ty + 16 * k, j = j0 + r, i = i0 + 4 * tx;
    if (i < H && j < W)
      store4(dst + static_cast<int64_t>(j) * H + i,
             make_float4(tile[4 * tx][r], tile[4 * tx + 1][r], tile[4 * tx + 2][r], tile[4 * tx + 3][r]));
  }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
ss2d_merge4_kernel(const float *yr, const float *__restrict__ yc, const T *__restrict__ z, T *out,
                   int H, int W, int tiles_w, float scale) {
  __shared__ float tile[kTile4][kTile4 + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile4, j0 = tj * kTile4;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float *c = yc + pl * H * W;
  const int64_t base = pl * H * W;
  float4 v[4], r4[4], z4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {                             // yc rows j, contiguous in i
    const int j = j0 + ty + 16 * k, i = i0 + 4 * tx;
    v[k] = (i < H && j < W) ? load4(c + static_cast<int64_t>(j) * H + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {                             // yr and z rows i, contiguous in j
    const int i = i0 + ty + 16 * k, j = j0 + 4 * tx;
    const bool ok = i < H && j < W;
    const int64_t e = base + static_cast<int64_t>(i) * W + j;
    r4[k] = ok ? load4(yr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    z4[k] = (ok && z != nullptr) ? load4(z + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float *t = &tile[ty + 16 * k][4 * tx];
    t[0] = v[k].x; t[1] = v[k].y; t[2] = v[k].z; t[3] = v[k].w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ty + 16 * k, i = i0 + r, j = j0 + 4 * tx;
    if (i < H && j < W) {
      const float cx = tile[4 * tx][r], cy = tile[4 * tx + 1][r], cz = tile[4 * tx + 2][r],
                  cw = tile[4 * tx + 3][r];
      float4 o = make_float4(scale * (r4[k].x + cx), scale * (r4[k].y + cy), scale * (r4[k].z + cz),
                             scale * (r4[k].w + cw));
      if (z != nullptr) {
        o.x *= silu_f(z4[k].x); o.y *= silu_f(z4[k].y); o.z *= silu_f(z4[k].z); o.w *= silu_f(z4[k].w);
      }
      store4(out + base + static_cast<int64_t>(i) * W + j, o);
    }
  }
}

// The gate's backward for the four-direction scan, writing the output
// gradient in both layouts the backward scans read: with y = yr[p][i][j] +
// yc[p][j][i] (the row and column traversals' sums), g = scale dout SiLU(z)
// goes to dy ([P][H][W]) and dyt ([P][W][H]), and dz = scale dout y SiLU'(z),
// SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z).  Without z, g = scale dout
// (yr, yc, dz unused).  64 x 64 tiles, four values per access, as the merge.
__global__ void __launch_bounds__(kThreads)
ss2d_gate_bwd4_kernel(const float *__restrict__ yr, const float *__restrict__ yc,
                      const float *__restrict__ z, const float *__restrict__ dout,
                      float *__restrict__ dy, float *__restrict__ dyt, float *__restrict__ dz,
                      int H, int W, int tiles_w, float scale) {
  __shared__ float tile[kTile4][kTile4 + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile4, j0 = tj * kTile4;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int64_t base = pl * H * W;
  float4 g4[4];
  if (z != nullptr) {
    float4 v[4], r4[4], z4[4], d4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {                           // yc rows j, contiguous in i
      const int j = j0 + ty + 16 * k, i = i0 + 4 * tx;
      v[k] = (i < H && j < W) ? load4(yc + base + static_cast<int64_t>(j) * H + i)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {                           // yr, z, dout rows i, contiguous in j
      const int i = i0 + ty + 16 * k, j = j0 + 4 * tx;
      const bool ok = i < H && j < W;
      const int64_t e = base + static_cast<int64_t>(i) * W + j;
      r4[k] = ok ? load4(yr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      z4[k] = ok ? load4(z + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      d4[k] = ok ? load4(dout + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float *t = &tile[ty + 16 * k][4 * tx];
      t[0] = v[k].x; t[1] = v[k].y; t[2] = v[k].z; t[3] = v[k].w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = ty + 16 * k, i = i0 + r, j = j0 + 4 * tx;
      const float yv[4] = {r4[k].x + tile[4 * tx][r], r4[k].y + tile[4 * tx + 1][r],
                           r4[k].z + tile[4 * tx + 2][r], r4[k].w + tile[4 * tx + 3][r]};
      const float zv[4] = {z4[k].x, z4[k].y, z4[k].z, z4[k].w};
      const float dv[4] = {d4[k].x, d4[k].y, d4[k].z, d4[k].w};
      float gy[4], gz[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float g = scale * dv[c];
        const float sg = hw_rcp(1.0f + hw_exp2(-zv[c] * kLog2e));
        gy[c] = g * zv[c] * sg;
        gz[c] = g * yv[c] * (sg * __builtin_fmaf(zv[c], 1.0f - sg, 1.0f));
      }
      g4[k] = make_float4(gy[0], gy[1], gy[2], gy[3]);
      if (i < H && j < W) {
        const int64_t e = base + static_cast<int64_t>(i) * W + j;
        store4(dy + e, g4[k]);
        store4(dz + e, make_float4(gz[0], gz[1], gz[2], gz[3]));
      }
    }
    __syncthreads();                                         // the tile is read before it is refilled
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = i0 + ty + 16 * k, j = j0 + 4 * tx;
      const int64_t e = base + static_cast<int64_t>(i) * W + j;
      const float4 d = (i < H && j < W) ? load4(dout + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      g4[k] = make_float4(scale * d.x, scale * d.y, scale * d.z, scale * d.w);
      if (i < H && j < W) store4(dy + e, g4[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float *t = &tile[ty + 16 * k][4 * tx];
    t[0] = g4[k].x; t[1] = g4[k].y; t[2] = g4[k].z; t[3] = g4[k].w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {                             // dyt rows j, contiguous in i
    const int r = ty + 16 * k, j = j0 + r, i = i0 + 4 * tx;
    if (i < H && j < W)
      store4(dyt + base + static_cast<int64_t>(j) * H + i,
             make_float4(tile[4 * tx][r], tile[4 * tx + 1][r], tile[4 * tx + 2][r], tile[4 * tx + 3][r]));
  }
}

// The map's gradient from the four traversals' ones:
// du[p][i][j] = (d0 + d1)[p][i][j] + (d2 + d3)[p][j][i], where d0, d1 are the
// row traversals' ([P][H][W]) and d2, d3 the column traversals' ([P][W][H]).
__global__ void __launch_bounds__(kThreads)
ss2d_du_sum4_kernel(const float *__restrict__ d0, const float *__restrict__ d1,
                    const float *__restrict__ d2, const float *__restrict__ d3,
                    float *__restrict__ du, int H, int W, int tiles_w) {
  __shared__ float tile[kTile4][kTile4 + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile4, j0 = tj * kTile4;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int64_t base = pl * H * W;
  float4 a4[4], b4[4], c4[4], e4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {                             // d2, d3 rows j, contiguous in i
    const int j = j0 + ty + 16 * k, i = i0 + 4 * tx;
    const bool ok = i < H && j < W;
    const int64_t e = base + static_cast<int64_t>(j) * H + i;
    c4[k] = ok ? load4(d2 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    e4[k] = ok ? load4(d3 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {                             // d0, d1 rows i, contiguous in j
    const int i = i0 + ty + 16 * k, j = j0 + 4 * tx;
    const bool ok = i < H && j < W;
    const int64_t e = base + static_cast<int64_t>(i) * W + j;
    a4[k] = ok ? load4(d0 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    b4[k] = ok ? load4(d1 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float *t = &tile[ty + 16 * k][4 * tx];
    t[0] = c4[k].x + e4[k].x; t[1] = c4[k].y + e4[k].y; t[2] = c4[k].z + e4[k].z; t[3] = c4[k].w + e4[k].w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ty + 16 * k, i = i0 + r, j = j0 + 4 * tx;
    if (i < H && j < W)
      store4(du + base + static_cast<int64_t>(i) * W + j,
             make_float4((a4[k].x + b4[k].x) + tile[4 * tx][r], (a4[k].y + b4[k].y) + tile[4 * tx + 1][r],
                         (a4[k].z + b4[k].z) + tile[4 * tx + 2][r], (a4[k].w + b4[k].w) + tile[4 * tx + 3][r]));
  }
}

// out[p][i][j] = scale * (yr[p][i][j] + yc[p][j][i]) * SiLU(z[p][i][j]):
// yr holds the row traversals' sum ([P][H][W], fp32, may be out itself),
// yc the column traversals' ([P][W][H], fp32).  z may be NULL.
template <typename T>
__global__ void __launch_bounds__(kThreads)
ss2d_merge_kernel(const float *yr, const float *__restrict__ yc, const T *__restrict__ z, T *out,
                  int H, int W, int tiles_w, float scale) {
  __shared__ float tile[kTile][kTile + 1];
  const int64_t pl = blockIdx.x;
  const int ti = blockIdx.y / tiles_w, tj = blockIdx.y - (blockIdx.y / tiles_w) * tiles_w;
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  const float *c = yc + pl * H * W;
  for (int r = ty; r < kTile; r += kThreads / kTile) {   // yc rows j, contiguous in i
    const int j = j0 + r, i = i0 + tx;
    if (i < H && j < W) tile[r][tx] = c[static_cast<int64_t>(j) * H + i];
  }
  __syncthreads();
  const int64_t base = pl * H * W;
  for (int r = ty; r < kTile; r += kThreads / kTile) {   // out rows i, contiguous in j
    const int i = i0 + r, j = j0 + tx;
    if (i < H && j < W) {
      const int64_t e = base + static_cast<int64_t>(i) * W + j;
      float v = scale * (yr[e] + tile[tx][r]);
      if (z != nullptr) v *= silu_f(to_f32(z[e]));
      out[e] = from_f32<T>(v);
    }
  }
}

// u[t] = SiLU(cb + sum_k w[k] x[t - 3 + k]) on each row (x outside the row
// is 0); reverse: the same in reversed order, u[t] = SiLU(cb + sum_k w[k]
// x[t + 3 - k]).  The [rows x L] tensor is processed as one flat array, so
// short rows do not leave threads idle: each thread computes kConvPer
// consecutive outputs from its own inputs plus the four before them
// (forward) or after them (reverse), which are its neighbour thread's and
// come from cache; taps that fall outside the element's row are masked.
// One integer division per thread locates its first element's row; the
// channel's weights are reloaded only when a row ends inside the thread's run.
constexpr int kConvPer = 8;

template <typename T>
__global__ void __launch_bounds__(kThreads)
conv1d_silu_kernel(const T *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
                   T *__restrict__ out, int64_t n, int64_t L, int64_t dim, int reverse, int vec) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kConvPer;
  if (e0 >= n) return;
  // xs[4 + j] = x[e0 + j]; xs[0..3] the four before (forward) or, with
  // reverse, xs[4 + kConvPer ..] the four after; 0 outside [0, n)
  float xs[kConvPer + 8];
  const int64_t lo = e0 - 4;
  if (vec && lo >= 0 && e0 + kConvPer + 4 <= n) {
#pragma unroll
    for (int q = 0; q < kConvPer + 8; q += 4) {
      const float4 v = load4(x + lo + q);
      xs[q] = v.x; xs[q + 1] = v.y; xs[q + 2] = v.z; xs[q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kConvPer + 8; ++q) {
      const int64_t e = lo + q;
      xs[q] = (e >= 0 && e < n) ? to_f32(x[e]) : 0.0f;
    }
  }
  int64_t t, d;
  if (n <= 0xffffffffll) {                                 // 32-bit division where it suffices
    const uint32_t r32 = static_cast<uint32_t>(e0) / static_cast<uint32_t>(L);
    t = static_cast<uint32_t>(e0) - r32 * static_cast<uint32_t>(L);
    d = r32 % static_cast<uint32_t>(dim);
  } else {
    const int64_t row = e0 / L;
    t = e0 - row * L;
    d = row % dim;
  }
  float w0 = w[4 * d], w1 = w[4 * d + 1], w2 = w[4 * d + 2], w3 = w[4 * d + 3];
  float b = cb != nullptr ? cb[d] : 0.0f;
  float res[kConvPer];
#pragma unroll
  for (int j = 0; j < kConvPer; ++j) {
    const float *c = xs + 4 + j;                           // x[e0 + j]
    float v = __builtin_fmaf(w3, c[0], b);
    if (!reverse) {
      v = __builtin_fmaf(w2, t >= 1 ? c[-1] : 0.0f, v);
      v = __builtin_fmaf(w1, t >= 2 ? c[-2] : 0.0f, v);
      v = __builtin_fmaf(w0, t >= 3 ? c[-3] : 0.0f, v);
    } else {
      v = __builtin_fmaf(w2, t + 1 < L ? c[1] : 0.0f, v);
      v = __builtin_fmaf(w1, t + 2 < L ? c[2] : 0.0f, v);
      v = __builtin_fmaf(w0, t + 3 < L ? c[3] : 0.0f, v);
    }
    res[j] = silu_f(v);
    if (++t == L && j + 1 < kConvPer) {                    // next element starts a new row
      t = 0;
      if (++d == dim) d = 0;
      w0 = w[4 * d]; w1 = w[4 * d + 1]; w2 = w[4 * d + 2]; w3 = w[4 * d + 3];
      b = cb != nullptr ? cb[d] : 0.0f;
    }
  }
  if (vec && e0 + kConvPer <= n) {
#pragma unroll
    for (int q = 0; q < kConvPer; q += 4)
      store4(out + e0 + q, make_float4(res[q], res[q + 1], res[q + 2], res[q + 3]));
  } else {
#pragma unroll
    for (int j = 0; j < kConvPer; ++j)
      if (e0 + j < n) out[e0 + j] = from_f32<T>(res[j]);
  }
}

__global__ void __launch_bounds__(kThreads)
to_f32_kernel(const bf16_t *__restrict__ src, float *__restrict__ dst, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * kThreads)
    dst[e] = to_f32(src[e]);
}

unsigned stream_grid(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 64;   // 64 workgroups per CU, grid-stride beyond
  return static_cast<unsigned>(g < cap ? g : cap);
}

// Backward of the conv + SiLU, one channel d per grid column and a chunk of
// batch rows per grid row.  For output t, v[t] = cb + sum_k w[k] x[t - 3 + k]
// (forward; reverse mirrors it: x[t + 3 - k]), u = SiLU(v), and with
// dv = du SiLU'(v), SiLU'(v) = s (1 + v (1 - s)), s = sigmoid(v):
//   dx[t] = sum_k w[k] dv[t + 3 - k]   (reverse: dv[t - 3 + k])
//   dw[k] = sum over rows and t of dv[t] x[t - 3 + k]   (reverse: x[t + 3 - k])
//   dcb = sum of dv.
// One element per thread and iteration, so that every load is coalesced;
// each element recomputes the four dv it needs from cached x and du (eight
// consecutive elements per thread, each dv evaluated once, measured 15 %
// slower for their strided loads).  The workgroup's sums of dw and dcb go
// to partial [chunk][d][5], which conv1d_silu_bwd_reduce_kernel adds over
// chunks in a fixed order.
template <typename T, bool REV>
__global__ void __launch_bounds__(kThreads)
conv1d_silu_bwd_kernel(const T *__restrict__ x, const float *__restrict__ w,
                       const float *__restrict__ cb, const float *__restrict__ du,
                       float *__restrict__ dx, float *__restrict__ partial, int64_t batch,
                       int64_t dim, int L, int rows_per_chunk) {
  constexpr int sgn = REV ? -1 : 1;          // taps lie at t - sgn (3 - k)
  __shared__ float red[5][kThreads / 64];
  const int64_t d = blockIdx.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * rows_per_chunk;
  const int nrows = static_cast<int>(batch - b0 < rows_per_chunk ? batch - b0 : rows_per_chunk);
  const int n = nrows * L;
  float wk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) wk[k] = w[d * 4 + k];
  const float bias = cb != nullptr ? cb[d] : 0.0f;
  float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};   // dw[0..3], dcb
  for (int e = threadIdx.x; e < n; e += kThreads) {
    const int rb = e / L, t = e - rb * L;
    const int64_t base = ((b0 + rb) * dim + d) * L;
    // xv[j] = x[t + sgn (j - 3)] for j = 0 .. 6 (0 outside the row)
    float xv[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int s = t + sgn * (j - 3);
      xv[j] = (s >= 0 && s < L) ? to_f32(x[base + s]) : 0.0f;
    }
    float dxv = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {           // output t' = t + sgn o reads x[t] through tap 3 - o
      const int tp = t + sgn * o;
      if (tp < 0 || tp >= L) continue;
      float v = bias;
#pragma unroll
      for (int k = 0; k < 4; ++k) v = __builtin_fmaf(wk[k], xv[o + k], v);
      const float sg = hw_rcp(1.0f + hw_exp2(-v * kLog2e));
      const float dv = du[base + tp] * (sg * __builtin_fmaf(v, 1.0f - sg, 1.0f));
      dxv = __builtin_fmaf(wk[3 - o], dv, dxv);
      if (o == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(dv, xv[k], acc[k]);
        acc[4] += dv;
      }
    }
    dx[base + t] = dxv;
  }
  // workgroup sums: within each wave, then across the four waves
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    float v = acc[q];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[q][wv] = v;
  }
  __syncthreads();
  if (threadIdx.x < 5) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) v += red[threadIdx.x][k];
    partial[(static_cast<int64_t>(blockIdx.y) * dim + d) * 5 + threadIdx.x] = v;
  }
}

// dw [dim, 4] and dcb [dim] (may be null) from the chunk partials, in chunk order.
__global__ void __launch_bounds__(kThreads)
conv1d_silu_bwd_reduce_kernel(const float *__restrict__ partial, float *__restrict__ dw,
                              float *__restrict__ dcb, int64_t dim, int nchunk) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;   // d * 5 + q
  if (i >= dim * 5) return;
  float v = 0.0f;
  for (int c = 0; c < nchunk; ++c) v += partial[static_cast<int64_t>(c) * dim * 5 + i];
  const int64_t d = i / 5;
  const int q = static_cast<int>(i - d * 5);
  if (q < 4) dw[d * 4 + q] = v;
  else if (dcb != nullptr) dcb[d] = v;
}

// Backward of repeat_gate_kernel, one workgroup per grid (row r): with
// g = scale dout,
//   dz[i, j] = g y[p] SiLU'(z[i, j]),  SiLU'(z) = sg (1 + z (1 - sg)),
//   dy[p]    = sum over the repeated axis of g SiLU(z)   (g without z),
// p = i (axis 0: the sum runs over j) or j (axis 1: over i).  The sums run
// in index order (deterministic).
template <typename T>
__global__ void __launch_bounds__(kThreads)
repeat_gate_bwd_kernel(const float *__restrict__ y, const T *__restrict__ z,
                       const T *__restrict__ dout, float *__restrict__ dy, float *__restrict__ dz,
                       int H, int W, int axis, float scale) {
  const int64_t r = blockIdx.x;
  const int64_t hw = static_cast<int64_t>(H) * W;
  const int Lp = axis == 0 ? H : W;
  const float *yr = y + r * Lp;
  const T *zr = z != nullptr ? z + r * hw : nullptr;
  const T *dr = dout + r * hw;
  float *dzr = dz != nullptr ? dz + r * hw : nullptr;
  float *dyr = dy + r * Lp;
  auto term = [&](int i, int j, float yp) __attribute__((always_inline)) {
    const int64_t e = static_cast<int64_t>(i) * W + j;
    const float g = scale * to_f32(dr[e]);
    if (zr == nullptr) return g;
    const float zv = to_f32(zr[e]);
    const float sg = hw_rcp(1.0f + hw_exp2(-zv * kLog2e));
    dzr[e] = g * yp * (sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f));
    return g * zv * sg;
  };
  if (axis == 0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = wave; i < H; i += kThreads / 64) {
      const float yp = yr[i];
      float acc = 0.0f;
      for (int j = lane; j < W; j += 64) acc += term(i, j, yp);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (lane == 0) dyr[i] = acc;
    }
  } else {
    for (int j = threadIdx.x; j < W; j += kThreads) {
      const float yp = yr[j];
      float acc = 0.0f;
      for (int i = 0; i < H; ++i) acc += term(i, j, yp);
      dyr[j] = acc;
    }
  }
}

// Backward of the mean pool: du[i, j] = dubar[p] inv (p = i for axis 0, j for
// axis 1), one workgroup per grid.
__global__ void __launch_bounds__(kThreads)
pool_bwd_kernel(const float *__restrict__ dubar, float *__restrict__ du, int H, int W, int axis,
                float inv) {
  const int64_t r = blockIdx.x;
  const int Lp = axis == 0 ? H : W;
  const float *dr = dubar + r * Lp;
  float *o = du + r * static_cast<int64_t>(H) * W;
  Walk w;
  w.init(threadIdx.x, W);
  for (int e = threadIdx.x; e < H * W; e += kThreads, w.next())
    o[e] = dr[axis == 0 ? w.a : w.b] * inv;
}

bool aligned(const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

hipError_t launch_atrous_gather(const void *x, void *streams, int64_t batch, int64_t ch,
                                int64_t H, int64_t W, bool bf16, hipStream_t s) {
  const int64_t planes = batch * ch;
  if (planes == 0) return hipSuccess;
  const int64_t Lg = ((H + 1) / 2) * ((W + 1) / 2);
  const uintptr_t va = bf16 ? 8 : 16;
  // vec 1: rows that are multiples of 4 values; vec 2: any rows, chunked
  // (aligned tensors, the staged plane with room for the chunks' margins)
  const bool al = aligned(x, va) && aligned(streams, va);
  int vec = (H * W <= kPlaneLds) && (H * W) % 4 == 0 && Lg % 4 == 0 && al ? 1 : 0;
  if (vec == 0 && H * W + 8 <= kPlaneLds && al && planes * H * W < (int64_t{1} << 31)) vec = 2;
  const int staged = (vec != 0 || H * W <= kPlaneLds) ? 1 : 0;
  const size_t lds = staged ? static_cast<size_t>(H * W + 8) * (bf16 ? 2 : 4) : 0;
  if (bf16)
    hipLaunchKernelGGL(atrous_gather_kernel<bf16_t>, dim3(planes), dim3(kThreads), lds, s,
                       static_cast<const bf16_t *>(x), static_cast<bf16_t *>(streams), ch,
                       static_cast<int>(H), static_cast<int>(W), staged, vec);
  else
    hipLaunchKernelGGL(atrous_gather_kernel<float>, dim3(planes), dim3(kThreads), lds, s,
                       static_cast<const float *>(x), static_cast<float *>(streams), ch,
                       static_cast<int>(H), static_cast<int>(W), staged, vec);
  return hipGetLastError();
}

hipError_t launch_atrous_scatter(const void *streams, void *y, int64_t batch, int64_t ch,
                                 int64_t H, int64_t W, bool bf16, hipStream_t s) {
  const int64_t planes = batch * ch;
  if (planes == 0) return hipSuccess;
  const int64_t Lg = ((H + 1) / 2) * ((W + 1) / 2);
  const uintptr_t va = bf16 ? 8 : 16;
  const bool al = aligned(streams, va) && aligned(y, va);
  const int64_t SL = (Lg + 3) / 4 * 4 + 4;              // the chunked path's LDS slot per stream
  int vec = (4 * Lg <= kPlaneLds) && Lg % 4 == 0 && W % 4 == 0 && al ? 1 : 0;
  if (vec == 0 && 4 * SL <= kPlaneLds && al && planes * 4 * Lg < (int64_t{1} << 31)) vec = 2;
  const int staged = (vec != 0 || 4 * Lg <= kPlaneLds) ? 1 : 0;
  const size_t lds = staged ? static_cast<size_t>(4 * SL) * (bf16 ? 2 : 4) : 0;
  if (bf16)
    hipLaunchKernelGGL(atrous_scatter_kernel<bf16_t>, dim3(planes), dim3(kThreads), lds, s,
                       static_cast<const bf16_t *>(streams), static_cast<bf16_t *>(y), ch,
                       static_cast<int>(H), static_cast<int>(W), staged, vec);
  else
    hipLaunchKernelGGL(atrous_scatter_kernel<float>, dim3(planes), dim3(kThreads), lds, s,
                       static_cast<const float *>(streams), static_cast<float *>(y), ch,
                       static_cast<int>(H), static_cast<int>(W), staged, vec);
  return hipGetLastError();
}


// The four-wide transpose and merge read and write rows of both orientations
// four at a time: H and W multiples of 4, planes aligned to four elements.
bool tile4_ok(int64_t H, int64_t W, std::initializer_list<const void *> ptrs, bool bf16) {
  if (H % 4 != 0 || W % 4 != 0) return false;
  for (const void *p : ptrs)
    if (!aligned(p, bf16 ? 8 : 16)) return false;
  return true;
}

// Four-wide accesses need W % 4 == 0, aligned rows, and (for the lane
// reduction and the LDS combine) W / 4 a power of two no larger than 64.
int vec_ok(const void *a, const void *b, const void *c, int64_t W, bool bf16) {
  const uintptr_t al = bf16 ? 8 : 16;
  const int64_t q = W / 4;
  const bool pow2 = q > 0 && q <= 64 && (q & (q - 1)) == 0;
  return (W % 4 == 0 && pow2 && reinterpret_cast<uintptr_t>(a) % al == 0 &&
          reinterpret_cast<uintptr_t>(b) % al == 0 && reinterpret_cast<uintptr_t>(c) % 16 == 0)
             ? 1 : 0;
}

hipError_t launch_mean_pool(const void *u, float *pooled, int64_t rows, int64_t H, int64_t W,
                            int axis, bool bf16, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const float inv = static_cast<float>(1.0 / static_cast<double>(axis == 0 ? W : H));
  const int vec = vec_ok(u, u, pooled, W, bf16);
  if (bf16)
    hipLaunchKernelGGL(mean_pool_kernel<bf16_t>, dim3(rows), dim3(kThreads), 0, s,
                       static_cast<const bf16_t *>(u), pooled, static_cast<int>(H),
                       static_cast<int>(W), axis, inv, vec);
  else
    hipLaunchKernelGGL(mean_pool_kernel<float>, dim3(rows), dim3(kThreads), 0, s,
                       static_cast<const float *>(u), pooled, static_cast<int>(H),
                       static_cast<int>(W), axis, inv, vec);
  return hipGetLastError();
}

hipError_t launch_repeat_gate(const float *y, const void *z, void *out, int64_t rows, int64_t H,
                              int64_t W, int axis, float scale, bool bf16, hipStream_t s) {
  if (rows * H * W == 0) return hipSuccess;
  const int vec = vec_ok(z != nullptr ? z : out, out, y, W, bf16) &&
                  (axis == 0 || (W * 4) % 16 == 0);
  if (bf16)
    hipLaunchKernelGGL(repeat_gate_kernel<bf16_t>, dim3(static_cast<unsigned>(rows)), dim3(kThreads),
                       0, s, y, static_cast<const bf16_t *>(z), static_cast<bf16_t *>(out),
                       static_cast<int>(H), static_cast<int>(W), axis, scale, vec);
  else
    hipLaunchKernelGGL(repeat_gate_kernel<float>, dim3(static_cast<unsigned>(rows)), dim3(kThreads),
                       0, s, y, static_cast<const float *>(z), static_cast<float *>(out),
                       static_cast<int>(H), static_cast<int>(W), axis, scale, vec);
  return hipGetLastError();
}

hipError_t launch_repeat_gate_bwd(const float *y, const void *z, const void *dout, float *dy, float *dz,
                                  int64_t rows, int64_t H, int64_t W, int axis, float scale, bool bf16,
                                  hipStream_t s) {
  if (rows * H * W == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(repeat_gate_bwd_kernel<bf16_t>, dim3(static_cast<unsigned>(rows)), dim3(kThreads),
                       0, s, y, static_cast<const bf16_t *>(z), static_cast<const bf16_t *>(dout), dy, dz,
                       static_cast<int>(H), static_cast<int>(W), axis, scale);
  else
    hipLaunchKernelGGL(repeat_gate_bwd_kernel<float>, dim3(static_cast<unsigned>(rows)), dim3(kThreads),
                       0, s, y, static_cast<const float *>(z), static_cast<const float *>(dout), dy, dz,
                       static_cast<int>(H), static_cast<int>(W), axis, scale);
  return hipGetLastError();
}

hipError_t launch_pool_bwd(const float *dubar, float *du, int64_t rows, int64_t H, int64_t W, int axis,
                           hipStream_t s) {
  if (rows * H * W == 0) return hipSuccess;
  const float inv = static_cast<float>(1.0 / static_cast<double>(axis == 0 ? W : H));
  hipLaunchKernelGGL(pool_bwd_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, s, dubar, du,
                     static_cast<int>(H), static_cast<int>(W), axis, inv);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *in, void *out, int64_t planes, int64_t H, int64_t W, bool bf16,
                            hipStream_t s) {
  if (planes * H * W == 0) return hipSuccess;
  if (tile4_ok(H, W, {in, out}, bf16)) {
    const int th = static_cast<int>((H + kTile4 - 1) / kTile4), tw = static_cast<int>((W + kTile4 - 1) / kTile4);
    const dim3 grid(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw));
    if (bf16)
      hipLaunchKernelGGL(transpose4_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                         static_cast<const bf16_t *>(in), static_cast<bf16_t *>(out),
                         static_cast<int>(H), static_cast<int>(W), tw);
    else
      hipLaunchKernelGGL(transpose4_kernel<float>, grid, dim3(kThreads), 0, s,
                         static_cast<const float *>(in), static_cast<float *>(out),
                         static_cast<int>(H), static_cast<int>(W), tw);
    return hipGetLastError();
  }
  const int th = static_cast<int>((H + kTile - 1) / kTile), tw = static_cast<int>((W + kTile - 1) / kTile);
  const dim3 grid(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw));
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t *>(in), static_cast<bf16_t *>(out),
                       static_cast<int>(H), static_cast<int>(W), tw);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float *>(in), static_cast<float *>(out),
                       static_cast<int>(H), static_cast<int>(W), tw);
  return hipGetLastError();
}

bool ss2d_tile4_ok(int64_t H, int64_t W, std::initializer_list<const void *> ptrs) {
  return tile4_ok(H, W, ptrs, false);
}

hipError_t launch_ss2d_gate_bwd(const float *yr, const float *yc, const float *z, const float *dout,
                                float *dy, float *dyt, float *dz, int64_t planes, int64_t H, int64_t W,
                                float scale, hipStream_t s) {
  if (planes * H * W == 0) return hipSuccess;
  if (!tile4_ok(H, W, {yr, yc, z, dout, dy, dyt, dz}, false)) return hipErrorInvalidValue;
  const int th = static_cast<int>((H + kTile4 - 1) / kTile4), tw = static_cast<int>((W + kTile4 - 1) / kTile4);
  hipLaunchKernelGGL(ss2d_gate_bwd4_kernel, dim3(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw)),
                     dim3(kThreads), 0, s, yr, yc, z, dout, dy, dyt, dz, static_cast<int>(H),
                     static_cast<int>(W), tw, scale);
  return hipGetLastError();
}

hipError_t launch_ss2d_du_sum(const float *d0, const float *d1, const float *d2, const float *d3,
                              float *du, int64_t planes, int64_t H, int64_t W, hipStream_t s) {
  if (planes * H * W == 0) return hipSuccess;
  if (!tile4_ok(H, W, {d0, d1, d2, d3, du}, false)) return hipErrorInvalidValue;
  const int th = static_cast<int>((H + kTile4 - 1) / kTile4), tw = static_cast<int>((W + kTile4 - 1) / kTile4);
  hipLaunchKernelGGL(ss2d_du_sum4_kernel, dim3(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw)),
                     dim3(kThreads), 0, s, d0, d1, d2, d3, du, static_cast<int>(H), static_cast<int>(W), tw);
  return hipGetLastError();
}

hipError_t launch_ss2d_merge(const float *yr, const float *yc, const void *z, void *out,
                             int64_t planes, int64_t H, int64_t W, float scale, bool bf16,
                             hipStream_t s) {
  if (planes * H * W == 0) return hipSuccess;
  if (tile4_ok(H, W, {yr, yc}, false) && tile4_ok(H, W, {out}, bf16) &&
      (z == nullptr || aligned(z, bf16 ? 8 : 16))) {
    const int th = static_cast<int>((H + kTile4 - 1) / kTile4), tw = static_cast<int>((W + kTile4 - 1) / kTile4);
    const dim3 grid(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw));
    if (bf16)
      hipLaunchKernelGGL(ss2d_merge4_kernel<bf16_t>, grid, dim3(kThreads), 0, s, yr, yc,
                         static_cast<const bf16_t *>(z), static_cast<bf16_t *>(out),
                         static_cast<int>(H), static_cast<int>(W), tw, scale);
    else
      hipLaunchKernelGGL(ss2d_merge4_kernel<float>, grid, dim3(kThreads), 0, s, yr, yc,
                         static_cast<const float *>(z), static_cast<float *>(out),
                         static_cast<int>(H), static_cast<int>(W), tw, scale);
    return hipGetLastError();
  }
  const int th = static_cast<int>((H + kTile - 1) / kTile), tw = static_cast<int>((W + kTile - 1) / kTile);
  const dim3 grid(static_cast<unsigned>(planes), static_cast<unsigned>(th * tw));
  if (bf16)
    hipLaunchKernelGGL(ss2d_merge_kernel<bf16_t>, grid, dim3(kThreads), 0, s, yr, yc,
                       static_cast<const bf16_t *>(z), static_cast<bf16_t *>(out),
                       static_cast<int>(H), static_cast<int>(W), tw, scale);
  else
    hipLaunchKernelGGL(ss2d_merge_kernel<float>, grid, dim3(kThreads), 0, s, yr, yc,
                       static_cast<const float *>(z), static_cast<float *>(out),
                       static_cast<int>(H), static_cast<int>(W), tw, scale);
  return hipGetLastError();
}

hipError_t launch_conv1d_silu(const void *x, const float *w, const float *cb, void *out,
                              int64_t rows, int64_t L, int64_t dim, int reverse, bool bf16,
                              hipStream_t s) {
  const int64_t n = rows * L;
  if (n == 0) return hipSuccess;
  const int64_t per_block = static_cast<int64_t>(kConvPer) * kThreads;
  const dim3 grid(static_cast<unsigned>((n + per_block - 1) / per_block));
  const int vec = aligned(out, bf16 ? 8 : 16) && aligned(x, bf16 ? 8 : 16) ? 1 : 0;
  if (bf16)
    hipLaunchKernelGGL(conv1d_silu_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t *>(x), w, cb, static_cast<bf16_t *>(out), n, L, dim,
                       reverse, vec);
  else
    hipLaunchKernelGGL(conv1d_silu_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float *>(x), w, cb, static_cast<float *>(out), n, L, dim,
                       reverse, vec);
  return hipGetLastError();
}

int conv1d_bwd_chunks(int64_t batch, int64_t dim, int *rows_per_chunk) {
  // enough workgroups to fill the chip: about 2048 of them
  int64_t nchunk = (2048 + dim - 1) / dim;
  if (nchunk > batch) nchunk = batch;
  if (nchunk < 1) nchunk = 1;
  const int64_t rpc = (batch + nchunk - 1) / nchunk;
  *rows_per_chunk = static_cast<int>(rpc);
  return static_cast<int>((batch + rpc - 1) / rpc);
}

hipError_t launch_conv1d_silu_bwd(const void *x, const float *w, const float *cb, const float *du,
                                  float *dx, float *dw, float *dcb, float *partial, int64_t batch,
                                  int64_t dim, int64_t L, int reverse, bool bf16, hipStream_t s) {
  if (batch * dim * L == 0) return hipSuccess;
  int rpc = 0;
  const int nchunk = conv1d_bwd_chunks(batch, dim, &rpc);
  const dim3 grid(static_cast<unsigned>(dim), static_cast<unsigned>(nchunk));
  const int Li = static_cast<int>(L);
  if (bf16 && reverse)
    hipLaunchKernelGGL((conv1d_silu_bwd_kernel<bf16_t, true>), grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t *>(x), w, cb, du, dx, partial, batch, dim, Li, rpc);
  else if (bf16)
    hipLaunchKernelGGL((conv1d_silu_bwd_kernel<bf16_t, false>), grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t *>(x), w, cb, du, dx, partial, batch, dim, Li, rpc);
  else if (reverse)
    hipLaunchKernelGGL((conv1d_silu_bwd_kernel<float, true>), grid, dim3(kThreads), 0, s,
                       static_cast<const float *>(x), w, cb, du, dx, partial, batch, dim, Li, rpc);
  else
    hipLaunchKernelGGL((conv1d_silu_bwd_kernel<float, false>), grid, dim3(kThreads), 0, s,
                       static_cast<const float *>(x), w, cb, du, dx, partial, batch, dim, Li, rpc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nred = dim * 5;
  hipLaunchKernelGGL(conv1d_silu_bwd_reduce_kernel, dim3(static_cast<unsigned>((nred + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, partial, dw, dcb, dim, nchunk);
  return hipGetLastError();
}

hipError_t launch_to_f32(const void *src, float *dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(to_f32_kernel, dim3(stream_grid(n)), dim3(kThreads), 0, s,
                     static_cast<const bf16_t *>(src), dst, n);
  return hipGetLastError();
}

}  // namespace vmk
