// Order keys and lane reductions shared by the top-K selections: logits
// become 32-bit keys whose unsigned order is the float order (-0.0 folded
// onto +0.0; key 0 lies below every logit and marks a removed or absent
// column), and segments of S lanes of a wave take their max or min key with
// DPP row operations.
#pragma once
#include "common.hpp"

namespace route {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// Lane permutation inside rows of 16 (every lane reads a lane of its own row,
// so the bound control never applies; it lets the move fold into the max/min).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, true));
}

constexpr int kDppXor1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i inside each 16

// Max over each aligned segment of S lanes; every lane of the segment gets it.
template <int S>
__device__ __forceinline__ uint32_t seg_max(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  if (S >= 8) v = max(v, dpp<kDppHalfMirror>(v));
  if (S >= 16) v = max(v, dpp<kDppMirror>(v));
  if (S == 32) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16, kWave)));
  if (S == 64) {
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    v = max(max(a, b), max(c, d));
  }
  return v;
}

// Min over each aligned segment of S >= 16 lanes; every lane of the segment gets it.
template <int S>
__device__ __forceinline__ uint32_t seg_min(uint32_t v) {
  v = min(v, dpp<kDppXor1>(v));
  v = min(v, dpp<kDppXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  if (S == 32) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16, kWave)));
  if (S == 64) {
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    v = min(min(a, b), min(c, d));
  }
  return v;
}

// Top-K of one row held by an aligned segment of S lanes (S >= 16), V values
// per lane: lane s holds columns s + S v, their order keys in key[] (0 for an
// absent column, whose value must then be -inf). Picks go in the library's
// order, larger key first and the lower column on equal keys; each round
// takes the segment's best key, the lowest column holding it, and clears it.
// K (<= kMaxK) may vary at run time. On return lane s < K of the segment
// holds pick s: its column and its softmax weight, over the K picks
// (renorm) or over every present column (renorm = 0). The arithmetic is the
// fixed-shape top-K kernel's with one group, so the results are the same
// bits.
template <int S, int V>
__device__ __forceinline__ void seg_topk(const float (&val)[V], uint32_t (&key)[V], int K,
                                         int renorm, int* col, float* weight) {
  const int s = lane_id() & (S - 1);
  float mysel = 0.f, top = 0.f;
  int mycol = 0;
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r >= K) break;
    uint32_t best = 0u;
    int bv = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (key[v] > best) {  // strict: lowest v on equal keys
        best = key[v];
        bv = v;
      }
    }
    const uint32_t m = seg_max<S>(best);
    const int c =
        static_cast<int>(seg_min<S>(best == m ? static_cast<uint32_t>(s + S * bv) : 0xffffffffu));
    const bool mine = s == (c & (S - 1));
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = (mine && bv == v) ? 0u : key[v];
    if (r == 0) top = key_float(m);
    if (s == r) {
      mysel = key_float(m);
      mycol = c;
    }
  }
  float w;
  if (renorm) {
    const float e = s < K ? __expf(mysel - top) : 0.f;
    float z = e;
#pragma unroll
    for (int o = S / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, kWave);
    w = __fdividef(e, z);
  } else {
    float zl = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) zl += __expf(val[v] - top);
#pragma unroll
    for (int o = S / 2; o > 0; o >>= 1) zl += __shfl_xor(zl, o, kWave);
    w = __fdividef(__expf(mysel - top), zl);
  }
  *col = mycol;
  *weight = w;
}

}  // namespace route
