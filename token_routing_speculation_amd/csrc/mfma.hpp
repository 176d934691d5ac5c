// bf16 matrix-core products shared by the kernels that use them.
// v_mfma_f32_16x16x32_bf16, D = A . B + C for a 16 x 32 A fragment and a
// 32 x 16 B fragment. Lane l holds row (A) or column (B) l % 16, elements
// k = 8 (l / 16) .. 8 (l / 16) + 7 as one 16-byte vector; the result holds
// rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
#pragma once
#include "common.hpp"

namespace route {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16, D = A . B + C for a 32 x 16 A fragment and a
// 16 x 32 B fragment: lane l holds row (A) or column (B) l % 32 and eight
// consecutive k, the halves l / 32 = 0, 1 taking the two 8-wide k halves (any
// consistent assignment of k to lanes gives the same product); the result
// holds column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4 for e = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One 16-byte piece per lane from global memory into LDS: lane i writes at
// lds_base + 16 i (lds_base is wave-uniform). Completion is counted by vmcnt.
__device__ __forceinline__ void lds_load16(const void* g, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
#endif
}

// Waits until at most N of this wave's vector-memory operations are pending
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits for this wave's LDS (and scalar memory) operations.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Keeps the compiler from moving memory accesses across this point (the
// bare barrier below does not order them by itself).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier after this wave's LDS writes have completed, without the
// full fence of __syncthreads (which also waits for every pending global
// load): the caller waits for whatever else the other waves must see.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

}  // namespace route
