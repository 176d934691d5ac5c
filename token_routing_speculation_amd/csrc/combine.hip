// moe_combine: weighted combine of expert outputs with the SAG unshuffle.
// "Speculative MoE" notes, section 1 (combine brings the K expert outputs
// back to the token and sums them with the gate weights) and section 3.1
// (SAG returns each shuffled token to its original row: out_row). In the
// FoE layout the K slots span the H groups, so the sum is also the
// cross-group sum ("Federation of Experts (FoE)" article).
//
// One wave per token: K row gathers of 16-byte vectors, binary32 FMA in slot
// order k = 0..K-1, one row store (bf16 nearest-even or float32). The
// unshuffle comes in two forms with the same results: moe_combine scatters
// (wave j writes row out_row[j]), moe_combine_gather gathers (wave t writes
// row t, combining token in_row[t]). The gather form writes its rows in
// order; measured at the DeepSeek-V2 shape (16384 rows of 5120, K = 6,
// graph replay), a random row permutation costs the scattered stores 17 us
// of 229 us, while the gathers go to scattered rows either way.
//
// Both the gathers and the row stores are streaming (nontemporal): neither is re-read
// within the pass, and a streaming store leaves MI355X's memory-side cache to
// the activations that the shuffle writes and the gate and the dispatch read
// back. Measured on whole DeepSeek-V2-shaped passes, that keeps about 40 us
// of HBM reads per pass out of the following stages; with plain stores the
// combine alone moves the same bytes as fast (5.6 TB/s), but the pass does not.
#include "common.hpp"

namespace route {

constexpr int kCombThreads = 256;
constexpr int kCombGroup = 2;         // 16-byte vectors per lane gathered per step
constexpr bool kCombPingPong = true;  // next step's gathers issued before this step's stores

// Stores the combined vector v of a row (bf16 or float32 output).
template <int OUT_F32>
__device__ __forceinline__ void store_out(void* out, int64_t dst, int d, int v, const float* acc) {
  if (OUT_F32) {
    float* o = static_cast<float*>(out) + static_cast<size_t>(dst) * d + 8 * v;
    st16_stream(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                         __float_as_uint(acc[2]), __float_as_uint(acc[3])});
    st16_stream(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                             __float_as_uint(acc[6]), __float_as_uint(acc[7])});
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(dst) * d + 8 * v;
    st16_stream(o, pack8_cvt(acc));
  }
}

// Reads this token's K slots and weights; a slot out of range contributes
// nothing (weight 0, gathers row 0) and is flagged.
template <int KM>
__device__ __forceinline__ bool read_slots(const int* __restrict__ slot_of_pair,
                                           const float* __restrict__ weights, int64_t j, int K,
                                           int64_t nslots, int* slot, float* wk) {
  bool bad = false;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    slot[k] = 0;
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
  return bad;
}

// Token j of wave w and the row it goes to: j = w and row out_row[j] (or j)
// in the scatter form, j = in_row[w] and row w in the gather form. False
// (flagged) when the map points out of range: the row is skipped.
__device__ __forceinline__ bool token_and_row(int64_t w, int64_t n, const int* __restrict__ out_row,
                                              const int* __restrict__ in_row, int64_t* j,
                                              int64_t* dst, uint32_t* err) {
  *j = w;
  *dst = w;
  const int* map = in_row ? in_row : out_row;
  if (map) {
    const int64_t m = map[w];
    if (m < 0 || m >= n) {
      set_err(err, ROUTE_EBIT_INDEX_RANGE);
      return false;
    }
    *(in_row ? j : dst) = m;
  }
  return true;
}

// One wave per token, K a compile-time constant and CPL 16-byte vectors per
// lane. The row is processed in groups of two vectors; the gathers of the
// next group are issued before the stores of the current one (loads and
// stores share one in-order completion counter), from a ping-pong register
// set indexed statically so nothing is copied.
template <int KT, int CPL, int OUT_F32>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ weights,
    const int* __restrict__ slot_of_pair, int64_t n, int d, const int* __restrict__ out_row,
    const int* __restrict__ in_row, void* __restrict__ out, uint32_t* err) {
  constexpr int GV = kCombGroup < CPL ? kCombGroup : CPL;  // vectors per group
  constexpr int NG = (CPL + GV - 1) / GV;                   // groups per lane
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kCombThreads / kWave) + wave_id();
  if (w >= n) return;
  int64_t j, dst;
  if (!token_and_row(w, n, out_row, in_row, &j, &dst, err)) return;
  int slot[KT];
  float wk[KT];
  const bool bad = read_slots<KT>(slot_of_pair, weights, j, KT, n * KT, slot, wk);
  if (bad && lane_id() == 0) set_err(err, ROUTE_EBIT_INDEX_RANGE);
  const int lane = lane_id();
  const int nv = d >> 3;
  u32x4 buf[kCombPingPong ? 2 : 1][KT][GV];
  auto gather = [&](u32x4 (&b)[KT][GV], int g) {
#pragma unroll
    for (int q = 0; q < GV; ++q) {
      const int v = lane + (g * GV + q) * kWave;
      const int vv = v < nv ? v : 0;  // past the row end: reload vector 0, never stored
#pragma unroll
      for (int k = 0; k < KT; ++k)
        b[k][q] = ld16_stream(y + static_cast<size_t>(slot[k]) * d + 8 * vv);
    }
  };
  auto finish = [&](const u32x4 (&b)[KT][GV], int g) {
#pragma unroll
    for (int q = 0; q < GV; ++q) {
      const int v = lane + (g * GV + q) * kWave;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        float f[8];
        unpack8(b[k][q], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk[k], f[e], acc[e]);
      }
      if (v < nv) store_out<OUT_F32>(out, dst, d, v, acc);
    }
  };
  if (kCombPingPong) {
    gather(buf[0], 0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) gather(buf[(g + 1) & 1], g + 1);
      finish(buf[g & 1], g);
    }
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      gather(buf[0], g);
      finish(buf[0], g);
    }
  }
}

// Any K and row length: a plain loop over the row.
template <int OUT_F32>
__global__ __launch_bounds__(kCombThreads) void combine_any(
    const uint16_t* __restrict__ y, const float* __restrict__ weights,
    const int* __restrict__ slot_of_pair, int64_t n, int K, int d,
    const int* __restrict__ out_row, const int* __restrict__ in_row, void* __restrict__ out,
    uint32_t* err) {
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kCombThreads / kWave) + wave_id();
  if (w >= n) return;
  int64_t j, dst;
  if (!token_and_row(w, n, out_row, in_row, &j, &dst, err)) return;
  int slot[kMaxK];
  float wk[kMaxK];
  const bool bad = read_slots<kMaxK>(slot_of_pair, weights, j, K, n * K, slot, wk);
  if (bad && lane_id() == 0) set_err(err, ROUTE_EBIT_INDEX_RANGE);
  const int nv = d >> 3;
  for (int v = lane_id(); v < nv; v += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k < K) {
        float f[8];
        unpack8(ld16_stream(y + static_cast<size_t>(slot[k]) * d + 8 * v), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk[k], f[e], acc[e]);
      }
    }
    store_out<OUT_F32>(out, dst, d, v, acc);
  }
}

template <int KT, int OUT_F32>
static bool launch_combine_k(int cpl, unsigned grid, hipStream_t s, const uint16_t* y,
                             const float* w, const int* sop, int64_t n, int d, const int* out_row,
                             const int* in_row, void* out, uint32_t* err) {
  switch (cpl) {
#define ROUTE_CC(c)                                                                              \
  case c:                                                                                        \
    combine_kernel<KT, c, OUT_F32><<<grid, kCombThreads, 0, s>>>(y, w, sop, n, d, out_row,      \
                                                                 in_row, out, err);             \
    return true;
    ROUTE_CC(1) ROUTE_CC(2) ROUTE_CC(4) ROUTE_CC(8) ROUTE_CC(10)
#undef ROUTE_CC
    default: return false;
  }
}

template <int OUT_F32>
static void launch_combine(int K, unsigned grid, hipStream_t s, const uint16_t* y,
                           const float* w, const int* sop, int64_t n, int d, const int* out_row,
                           const int* in_row, void* out, uint32_t* err) {
  const int need = (d / 8 + kWave - 1) / kWave;
  const int cpl = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 10 ? 10 : 0;
  bool done = false;
  if (K == 2)
    done = launch_combine_k<2, OUT_F32>(cpl, grid, s, y, w, sop, n, d, out_row, in_row, out, err);
  if (K == 6)
    done = launch_combine_k<6, OUT_F32>(cpl, grid, s, y, w, sop, n, d, out_row, in_row, out, err);
  if (K == 8)
    done = launch_combine_k<8, OUT_F32>(cpl, grid, s, y, w, sop, n, d, out_row, in_row, out, err);
  if (!done)
    combine_any<OUT_F32><<<grid, kCombThreads, 0, s>>>(y, w, sop, n, K, d, out_row, in_row, out,
                                                       err);
}

}  // namespace route

using namespace route;

// Host checks and launch shared by both forms (exactly one of out_row and
// in_row may be given).
static int combine_entry(const uint16_t* y, const float* weights, const int32_t* slot_of_pair,
                         int64_t n, int32_t K, int32_t d, const int32_t* out_row,
                         const int32_t* in_row, void* out, int32_t out_dtype, uint32_t* err,
                         hipStream_t s) {
  if (n < 0 || K < 1 || d < 8 || d % 8 != 0 || (out_dtype != 0 && out_dtype != 1))
    return ROUTE_ERR_SHAPE;
  if (n * static_cast<int64_t>(K) >= (int64_t(1) << 31)) return ROUTE_ERR_SHAPE;
  if (K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!y || !weights || !slot_of_pair || !out) return ROUTE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out)) return ROUTE_ERR_ALIGN;
  const unsigned grid = ceil_div(n, kCombThreads / kWave);
  if (out_dtype == 1)
    launch_combine<1>(K, grid, s, y, weights, slot_of_pair, n, d, out_row, in_row, out, err);
  else
    launch_combine<0>(K, grid, s, y, weights, slot_of_pair, n, d, out_row, in_row, out, err);
  return launch_status();
}

ROUTE_API int moe_combine(const uint16_t* y, const float* weights, const int32_t* slot_of_pair,
                          int64_t n, int32_t K, int32_t d, const int32_t* out_row, void* out,
                          int32_t out_dtype, uint32_t* err, hipStream_t s) {
  return combine_entry(y, weights, slot_of_pair, n, K, d, out_row, nullptr, out, out_dtype, err,
                       s);
}

ROUTE_API int moe_combine_gather(const uint16_t* y, const float* weights,
                                 const int32_t* slot_of_pair, int64_t n, int32_t K, int32_t d,
                                 const int32_t* in_row, void* out, int32_t out_dtype,
                                 uint32_t* err, hipStream_t s) {
  if (n > 0 && !in_row) return ROUTE_ERR_NULL;
  return combine_entry(y, weights, slot_of_pair, n, K, d, nullptr, in_row, out, out_dtype, err,
                       s);
}
