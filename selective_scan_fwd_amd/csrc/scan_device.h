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

}  // namespace
}  // namespace vmk
