// Device helpers shared by the scan kernels (forward and backward): DPP row
// broadcasts, scheduling ties for loaded values, and buffer-resource access
// with out-of-range masking.
#pragma once

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
// B/C values it is used with.
template <int J> __device__ __forceinline__ void fmac_row_bcast(float &y, float c, float h);
#define VM_FMAC_BCAST(J)                                                              \
  template <>                                                                         \
  __device__ __forceinline__ void fmac_row_bcast<J>(float &y, float c, float h) {     \
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #J " row_mask:0xf bank_mask:0xf"    \
        : "+v"(y)                                                                     \
        : "v"(c), "v"(h));                                                            \
  }
VM_FMAC_BCAST(0) VM_FMAC_BCAST(1) VM_FMAC_BCAST(2) VM_FMAC_BCAST(3)
VM_FMAC_BCAST(4) VM_FMAC_BCAST(5) VM_FMAC_BCAST(6) VM_FMAC_BCAST(7)
VM_FMAC_BCAST(8) VM_FMAC_BCAST(9) VM_FMAC_BCAST(10) VM_FMAC_BCAST(11)
VM_FMAC_BCAST(12) VM_FMAC_BCAST(13) VM_FMAC_BCAST(14) VM_FMAC_BCAST(15)
#undef VM_FMAC_BCAST

// Ties a loaded value to this point of the program: nothing computed from it
// can be scheduled earlier (next to its load), where the wait for the load
// would also wait for the loads issued after it.
__device__ __forceinline__ float pin(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
// The same for a computed offset, which then reaches the memory instruction
// as one register (no splitting of the access by the select that chose it).
__device__ __forceinline__ uint32_t pin_u(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Orders one wave's LDS accesses across its lanes: LDS reads after this
// point see what any lane of the wave wrote before it.  A wave's LDS
// instructions execute in order, so this emits no instruction; it keeps the
// compiler from moving LDS accesses across it, which single-lane semantics
// would allow wherever a lane's own addresses provably differ.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Buffer access.  Token tensors, B, C and the exchange rows are read
// and written through buffer resources (base address and byte size in
// scalar registers, a 32-bit byte offset per lane).  An offset at or past
// the size reads 0 and drops a store, so masked elements need neither a
// branch nor a select, and every lane issues the same memory instructions.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;   // past every resource (sizes < 2 GiB)

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
template <typename Tin> __device__ __forceinline__ float bload(Rsrc r, uint32_t off);
template <> __device__ __forceinline__ float bload<float>(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}
template <> __device__ __forceinline__ float bload<bf16_t>(Rsrc r, uint32_t off) {
  return to_f32(static_cast<bf16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0)));
}
template <typename Tin> __device__ __forceinline__ void bstore(Rsrc r, uint32_t off, float v);
template <> __device__ __forceinline__ void bstore<float>(Rsrc r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, static_cast<int>(off), 0, 0);
}
template <> __device__ __forceinline__ void bstore<bf16_t>(Rsrc r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(from_f32<bf16_t>(v)), r,
                                        static_cast<int>(off), 0, 0);
}
// The same with a wave-uniform byte offset added in the scalar operand.
template <typename Tin> __device__ __forceinline__ void bstore_s(Rsrc r, uint32_t off, uint32_t soff, float v);
template <> __device__ __forceinline__ void bstore_s<float>(Rsrc r, uint32_t off, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, static_cast<int>(off),
                                        static_cast<int>(soff), 0);
}
template <> __device__ __forceinline__ void bstore_s<bf16_t>(Rsrc r, uint32_t off, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(from_f32<bf16_t>(v)), r,
                                        static_cast<int>(off), static_cast<int>(soff), 0);
}
// Four consecutive fp32 values at a 16-byte aligned offset, in one access.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t off, const float (&v)[4]) {
  const u32x4_t x = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                     __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, static_cast<int>(off), 0, 0);
}
// Two consecutive fp32 values at an 8-byte aligned offset, in one access.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void bstore2(Rsrc r, uint32_t off, const float (&v)[2]) {
  const u32x2_t x = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1])};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, static_cast<int>(off), 0, 0);
}
// (The whole vector is reinterpreted: a bit cast of one element of an
// ext_vector value reads element 0 with this compiler.)
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void bload4(Rsrc r, uint32_t off, float (&v)[4]) {
  const f32x4_t x =
      __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}

// Zero-order-hold input coefficient ("Norm or Direction?" page, section 3,
// eq. 2, for diagonal A): k = expm1(x) / A for x = dt A, given x2 = x
// log2(e), a = 2^x2 and iA = 1 / A (0 where A = 0, whose x = 0 takes the
// series).  For |x| < 1/8 it is dt g(x), g(x) = expm1(x) / x from its Taylor
// series to x^4 (truncation below 5e-8 relative); above, (a - 1) / A, where
// the rounding of a costs at most about 5e-7 relative because |expm1(x)| is
// then at least 0.117.  Both are computed and one is selected.
constexpr float kZohThr2 = 0.125f * kLog2e;   // |x| < 1/8 in units of x2
__device__ __forceinline__ float zoh_coef(float dt, float x2, float a, float iA) {
  constexpr float c1 = kLn2 / 2, c2 = kLn2 * kLn2 / 6, c3 = kLn2 * kLn2 * kLn2 / 24,
                  c4 = kLn2 * kLn2 * kLn2 * kLn2 / 120;
  float g = __builtin_fmaf(x2, c4, c3);
  g = __builtin_fmaf(x2, g, c2);
  g = __builtin_fmaf(x2, g, c1);
  g = __builtin_fmaf(x2, g, 1.0f);
  const float k_small = g * dt;
  const float k_large = __builtin_fmaf(a, iA, -iA);
  return __builtin_fabsf(x2) < kZohThr2 ? k_small : k_large;
}

// dk/dA of that coefficient (k given): dt^2 g'(x), with g'(x) = 1/2 + x/3 +
// x^2/8 + x^3/30 + x^4/144 for |x| < 1/8 (truncation below 1e-7 relative);
// above, (dt a - k) / A, whose cancellation costs at most about 1e-5
// relative at the switch.  (dk/ddt is a itself.)
__device__ __forceinline__ float zoh_coef_dA(float dt, float x2, float a, float iA, float k) {
  constexpr float e1 = 0.5f, e2 = kLn2 / 3, e3 = kLn2 * kLn2 / 8, e4 = kLn2 * kLn2 * kLn2 / 30,
                  e5 = kLn2 * kLn2 * kLn2 * kLn2 / 144;
  float g = __builtin_fmaf(x2, e5, e4);
  g = __builtin_fmaf(x2, g, e3);
  g = __builtin_fmaf(x2, g, e2);
  g = __builtin_fmaf(x2, g, e1);
  const float d_small = g * (dt * dt);
  const float d_large = __builtin_fmaf(dt, a, -k) * iA;
  return __builtin_fabsf(x2) < kZohThr2 ? d_small : d_large;
}

}  // namespace
}  // namespace vmk
