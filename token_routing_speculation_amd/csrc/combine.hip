// moe_combine: weighted combine of expert outputs with the SAG unshuffle.
// "Speculative MoE" notes, section 1 (combine brings the K expert outputs
// back to the token and sums them with the gate weights) and section 3.1
// (SAG returns each shuffled token to its original row: out_row). In the
// FoE layout the K slots span the H groups, so the sum is also the
// cross-group sum ("Federation of Experts (FoE)" article).
//
// One wave per token: K row gathers of 16-byte vectors, binary32 FMA in slot
// order k = 0..K-1, one row store (bf16 nearest-even or float32).
#include "common.hpp"

namespace route {

constexpr int kCombThreads = 256;

template <int KT, int OUT_F32>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ weights,
    const int* __restrict__ slot_of_pair, int64_t n, int K_dyn, int d,
    const int* __restrict__ out_row, void* __restrict__ out, uint32_t* err) {
  constexpr int KM = KT > 0 ? KT : kMaxK;
  const int K = KT > 0 ? KT : K_dyn;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * (kCombThreads / kWave) + threadIdx.x / kWave;
  if (j >= n) return;
  const int64_t nslots = n * K;
  int slot[KM];
  float wk[KM];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    slot[k] = -1;
    wk[k] = 0.f;
    if (k < K) {
      const int sl = slot_of_pair[j * K + k];
      if (sl >= 0 && sl < nslots) {
        slot[k] = sl;
        wk[k] = weights[j * K + k];
      } else {
        bad = true;
      }
    }
  }
  int64_t dst = j;
  if (out_row) {
    dst = out_row[j];
    if (dst < 0 || dst >= n) {
      set_err(err, ROUTE_EBIT_INDEX_RANGE);
      return;
    }
  }
  if (bad && lane_id() == 0) set_err(err, ROUTE_EBIT_INDEX_RANGE);
  const int nv = d >> 3;
  for (int v = lane_id(); v < nv; v += kWave) {
    u32x4 x[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (k < K && slot[k] >= 0) x[k] = ld16(y + static_cast<size_t>(slot[k]) * d + 8 * v);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < K && slot[k] >= 0) {
        float f[8];
        unpack8(x[k], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk[k], f[e], acc[e]);
      }
    }
    if (OUT_F32) {
      float* o = static_cast<float*>(out) + static_cast<size_t>(dst) * d + 8 * v;
      st16_stream(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                           __float_as_uint(acc[2]), __float_as_uint(acc[3])});
      st16_stream(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                               __float_as_uint(acc[6]), __float_as_uint(acc[7])});
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(dst) * d + 8 * v;
      st16_stream(o, pack8(acc));
    }
  }
}

template <int OUT_F32>
static void launch_combine(int K, unsigned grid, hipStream_t s, const uint16_t* y,
                           const float* w, const int* sop, int64_t n, int d, const int* out_row,
                           void* out, uint32_t* err) {
  switch (K) {
#define ROUTE_K_CASE(k)                                                                       \
  case k:                                                                                     \
    combine_kernel<k, OUT_F32><<<grid, kCombThreads, 0, s>>>(y, w, sop, n, K, d, out_row, out, \
                                                            err);                            \
    break;
    ROUTE_K_CASE(1) ROUTE_K_CASE(2) ROUTE_K_CASE(4) ROUTE_K_CASE(6) ROUTE_K_CASE(8)
#undef ROUTE_K_CASE
    default:
      combine_kernel<0, OUT_F32><<<grid, kCombThreads, 0, s>>>(y, w, sop, n, K, d, out_row, out,
                                                               err);
      break;
  }
}

}  // namespace route

using namespace route;

ROUTE_API int moe_combine(const uint16_t* y, const float* weights, const int32_t* slot_of_pair,
                          int64_t n, int32_t K, int32_t d, const int32_t* out_row, void* out,
                          int32_t out_dtype, uint32_t* err, hipStream_t s) {
  if (n < 0 || K < 1 || d < 8 || d % 8 != 0 || (out_dtype != 0 && out_dtype != 1))
    return ROUTE_ERR_SHAPE;
  if (n * static_cast<int64_t>(K) >= (int64_t(1) << 31)) return ROUTE_ERR_SHAPE;
  if (K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!y || !weights || !slot_of_pair || !out) return ROUTE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out)) return ROUTE_ERR_ALIGN;
  const unsigned grid = ceil_div(n, kCombThreads / kWave);
  if (out_dtype == 1)
    launch_combine<1>(K, grid, s, y, weights, slot_of_pair, n, d, out_row, out, err);
  else
    launch_combine<0>(K, grid, s, y, weights, slot_of_pair, n, d, out_row, out, err);
  return launch_status();
}
