// Device and host helpers shared by the libroute.so translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "route.h"

#define ROUTE_API extern "C" __attribute__((visibility("default")))

namespace route {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxK = 16;
constexpr int kMaxClusters = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 codec
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 8 bf16 in a 16-byte vector <-> 8 floats
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// pack8 through the hardware conversion (v_cvt_pk_bf16_f32, round to nearest
// even): the same bits as pack8 for every non-NaN value, denormals included;
// a vector holding a NaN takes pack8 itself, so NaN still becomes 0x7FC0.
__device__ __forceinline__ u32x4 pack8_cvt(const float* f) {
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) nan |= f[i] != f[i];
  if (__builtin_expect(nan, 0)) return pack8(f);
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_v h = {static_cast<__bf16>(f[2 * i]), static_cast<__bf16>(f[2 * i + 1])};
    uint32_t w;
    __builtin_memcpy(&w, &h, 4);
    v[i] = w;
  }
  return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming variants: data touched once (hint the caches not to keep it).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ unsigned wave_sum_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave-wide integer sum, returned to every lane (DPP row reductions, then
// the four row sums combined through scalar reads).
__device__ __forceinline__ int wave_sum_dpp(int v) {
  // every lane of these patterns reads a lane of its own row, so the bound
  // control never applies; it lets the move fold into the add
  v += __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, true);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, true);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, true);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, true);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Index of this wave in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot prove threadIdx.x / 64 uniform by itself, and control flow
// or addresses derived from it would otherwise be treated as divergent.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// ------------------------------------------------------------------ host side
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ERR_HIP;
}

inline unsigned ceil_div(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace route
