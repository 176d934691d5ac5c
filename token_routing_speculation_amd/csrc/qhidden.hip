// route_qhidden: q_l = LN_{l+1}(d_l + r_l), "Speculating Experts Accelerates
// Inference for Mixture-of-Experts", technical summary item 2.A. One wave
// per row: the row (d <= 8192) is held in registers as 16-byte vectors, the
// mean and the centred variance are two wave reductions in binary32, and the
// normalised row is stored as bf16 (nearest even).
#include "common.hpp"

namespace route {

constexpr int kLnThreads = 256;

template <int CPL>  // 16-byte vectors per lane
__global__ __launch_bounds__(kLnThreads) void qhidden_kernel(
    const uint16_t* __restrict__ r, const float* __restrict__ dvec,
    const float* __restrict__ gamma, const float* __restrict__ beta, int64_t n, int d,
    float eps, uint16_t* __restrict__ q) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kLnThreads / kWave) + wave_id();
  if (i >= n) return;
  const int lane = lane_id();
  const int nv = d >> 3;
  const uint16_t* row = r + static_cast<size_t>(i) * d;
  float x[CPL][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) {
      unpack8(ld16_stream(row + 8 * v), x[c]);
      const float4 d0 = *reinterpret_cast<const float4*>(dvec + 8 * v);
      const float4 d1 = *reinterpret_cast<const float4*>(dvec + 8 * v + 4);
      x[c][0] += d0.x; x[c][1] += d0.y; x[c][2] += d0.z; x[c][3] += d0.w;
      x[c][4] += d1.x; x[c][5] += d1.y; x[c][6] += d1.z; x[c][7] += d1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += x[c][e];
    }
  }
  const float mean = wave_sum(sum) / static_cast<float>(d);
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
  const float var = wave_sum(ss) / static_cast<float>(d);
  const float inv = 1.0f / sqrtf(var + eps);
  uint16_t* out = q + static_cast<size_t>(i) * d;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    if (v < nv) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = (x[c][e] - mean) * inv;
        if (gamma) t *= gamma[8 * v + e];
        if (beta) t += beta[8 * v + e];
        y[e] = t;
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
