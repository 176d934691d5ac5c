// route_qhidden: q_l = LN_{l+1}(d_l + r_l), "Speculating Experts Accelerates
// Inference for Mixture-of-Experts", technical summary item 2.A. One wave
// per row: the row (d <= 8192) is held in registers as 16-byte vectors, the
// mean and the centred variance are two wave reductions in binary32, and the
// normalised row is stored as bf16 (nearest even). The block's eight rows
// share d_l, staged once in LDS (read from L2 per row it would be twice the
// row's own bytes); the row loads are unconditional (vectors past the row
// end reload vector 0 and are masked out), so they issue back to back.
#include "common.hpp"

#include <type_traits>

namespace route {

constexpr int kLnThreads = 512;
constexpr int kLnMaxD = 8192;

// Wave-wide float sum, every lane gets it: DPP row reductions, then the four
// row sums through scalar reads.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xf, 0xf, true));
  };
  v += dpp(v, std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + e);
}

template <int CPL>  // 16-byte vectors per lane
__global__ __launch_bounds__(kLnThreads) void qhidden_kernel(
    const uint16_t* __restrict__ r, const float* __restrict__ dvec,
    const float* __restrict__ gamma, const float* __restrict__ beta, int64_t n, int d,
    float eps, uint16_t* __restrict__ q) {
  __shared__ __attribute__((aligned(16))) float sd[kLnMaxD];
  for (int j = threadIdx.x * 4; j < d; j += kLnThreads * 4)
    *reinterpret_cast<float4*>(sd + j) = *reinterpret_cast<const float4*>(dvec + j);
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kLnThreads / kWave) + wave_id();
  if (i >= n) return;
  const int lane = lane_id();
  const int nv = d >> 3;
  const uint16_t* row = r + static_cast<size_t>(i) * d;
  u32x4 raw[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    raw[c] = ld16_stream(row + 8 * (v < nv ? v : 0));
  }
  float x[CPL][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    const int vv = v < nv ? v : 0;
    unpack8(raw[c], x[c]);
    const float4 d0 = *reinterpret_cast<const float4*>(sd + 8 * vv);
    const float4 d1 = *reinterpret_cast<const float4*>(sd + 8 * vv + 4);
    x[c][0] += d0.x; x[c][1] += d0.y; x[c][2] += d0.z; x[c][3] += d0.w;
    x[c][4] += d1.x; x[c][5] += d1.y; x[c][6] += d1.z; x[c][7] += d1.w;
    if (v < nv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += x[c][e];
    }
  }
  const float mean = wave_sum_f32(sum) / static_cast<float>(d);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = x[c][e] - mean;
        ss += t * t;
      }
    }
  }
  const float var = wave_sum_f32(ss) / static_cast<float>(d);
  const float inv = 1.0f / sqrtf(var + eps);
  uint16_t* out = q + static_cast<size_t>(i) * d;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (x[c][e] - mean) * inv;
      if (gamma) {
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * v);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * v + 4);
        y[0] *= g0.x; y[1] *= g0.y; y[2] *= g0.z; y[3] *= g0.w;
        y[4] *= g1.x; y[5] *= g1.y; y[6] *= g1.z; y[7] *= g1.w;
      }
      if (beta) {
        const float4 b0 = *reinterpret_cast<const float4*>(beta + 8 * v);
        const float4 b1 = *reinterpret_cast<const float4*>(beta + 8 * v + 4);
        y[0] += b0.x; y[1] += b0.y; y[2] += b0.z; y[3] += b0.w;
        y[4] += b1.x; y[5] += b1.y; y[6] += b1.z; y[7] += b1.w;
      }
      st16(out + 8 * v, pack8(y));
    }
  }
}

}  // namespace route

using namespace route;

ROUTE_API int route_qhidden(const uint16_t* r, const float* dvec, const float* gamma,
                            const float* beta, int64_t n, int32_t d, float eps, uint16_t* q,
                            hipStream_t s) {
  if (n < 0 || d < 8 || d % 8 != 0 || !(eps >= 0.f)) return ROUTE_ERR_SHAPE;
  if (d > 8192) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!r || !dvec || !q) return ROUTE_ERR_NULL;
  if (!aligned16(r) || !aligned16(q) || !aligned16(dvec)) return ROUTE_ERR_ALIGN;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return ROUTE_ERR_ALIGN;
  const unsigned grid = ceil_div(n, kLnThreads / kWave);
  const int nv = d / 8;
  if (nv <= 64)
    qhidden_kernel<1><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 128)
    qhidden_kernel<2><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 256)
    qhidden_kernel<4><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else if (nv <= 512)
    qhidden_kernel<8><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  else
    qhidden_kernel<16><<<grid, kLnThreads, 0, s>>>(r, dvec, gamma, beta, n, d, eps, q);
  return launch_status();
}
