// route_topk: softmax + top-K of each token's router logits, plain or
// grouped ("Federation of Experts (FoE)" article, grouped MoE block: group h
// takes its own top k/H among experts [h*E/H, (h+1)*E/H)).
//
// A token is handled by a segment of S lanes of one wave (S = 4..32, a power
// of two >= E, for E <= 32; S = 16 for E <= 256 and 64 beyond, lane s holding
// the V = E/S logits of columns s, s+S, ...: the work per token is about
// K (V + log S) lane steps, so small segments keep every lane busy). Logits become 32-bit orderable keys (the
// float bits with the sign folded so unsigned order is float order; -0.0 is
// folded onto +0.0 first). Each of the K rounds takes a segment-wide max of
// the keys with DPP row operations (quad permutes and row mirrors, no LDS
// traffic), then resolves equal keys to the lowest expert index with a
// ballot; the chosen key is then removed (set to 0, below every logit).
#include "common.hpp"
#include "topk.hpp"

namespace route {

constexpr int kTopkThreads = 256;

template <int S, int V>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits,
                                                            int64_t n, int E, int K, int H,
                                                            int renorm, int* __restrict__ idx,
                                                            float* __restrict__ wout) {
  const int lane = threadIdx.x & (kWave - 1);
  const int s = lane & (S - 1);
  const int seg_base = lane & ~(S - 1);
  const int64_t tok = (static_cast<int64_t>(blockIdx.x) * kTopkThreads + threadIdx.x) / S;
  const bool active = tok < n;  // inactive lanes still join the cross-lane steps
  const float* row = logits + (active ? tok : 0) * static_cast<int64_t>(E);

  uint32_t key[V];
  float val[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = s + S * v;
    val[v] = (active && c < E) ? row[c] : 0.f;
    key[v] = (active && c < E) ? order_key(val[v]) : 0u;  // 0: never chosen
  }

  const int eg = E / H;
  const int kg = K / H;
  float selv[kMaxK];
  int selc[kMaxK];
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r < K) {
      const int lo = (r / kg) * eg;
      const int hi = lo + eg;
      uint32_t best = 0u;
      int bcol = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int c = s + S * v;
        if (c >= lo && c < hi && key[v] > best) {  // strict: lowest v on equal keys
          best = key[v];
          bcol = c;
        }
      }
      const uint32_t m = seg_max<S>(best);
      const uint64_t tie = __ballot(best == m && best != 0u);
      int col;
      if (V == 1) {
        // one column per lane: the lowest tied lane of the segment holds the
        // lowest column
        const uint64_t mine = (tie >> seg_base) & (S == 64 ? ~0ull : ((1ull << S) - 1));
        col = __builtin_ctzll(mine);
      } else {
        // several columns per lane: the smallest column among the tied lanes
        col = static_cast<int>(seg_min<S>(best == m ? static_cast<uint32_t>(bcol) : 0xffffffffu));
      }
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (s + S * v == col) key[v] = 0u;
      selc[r] = col;
      selv[r] = key_float(m);
    }
  }

  float wt[kMaxK];
  if (renorm) {
    // softmax over each group's chosen logits; the group's first pick is its max
    float mg = 0.f, z = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
      if (r < K) {
        if (r % kg == 0) {
          mg = selv[r];
          z = 0.f;
        }
        wt[r] = expf(selv[r] - mg);
        z += wt[r];
        if (r % kg == kg - 1) {
          // close the group: r - kg + 1 .. r share z
#pragma unroll
          for (int q = 0; q < kMaxK; ++q)
            if (q <= r && q > r - kg) wt[q] = wt[q] / z;
        }
      }
    }
  } else {
    float mall = -INFINITY;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r)
      if (r < K && r % kg == 0) mall = fmaxf(mall, selv[r]);
    float zl = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = s + S * v;
      if (active && c < E) zl += expf(val[v] - mall);
    }
#pragma unroll
    for (int o = S / 2; o > 0; o >>= 1) zl += __shfl_xor(zl, o, kWave);
#pragma unroll
    for (int r = 0; r < kMaxK; ++r)
      if (r < K) wt[r] = expf(selv[r] - mall) / zl;
  }

  if (active && s == 0) {
    int* io = idx + tok * K;
    float* wo = wout ? wout + tok * K : nullptr;
#pragma unroll
    for (int r = 0; r < kMaxK; ++r) {
      if (r < K) {
        io[r] = selc[r];
        if (wo) wo[r] = wt[r];
      }
    }
  }
}

// The same selection with the shape fixed at compile time: E = S * V exactly,
// K picks, H groups. Group h owns columns [h E/H, (h+1) E/H); when that range
// is a multiple of S, lane s's value v (column s + S v) belongs to group
// S v / (E/H) for every lane, so each round scans only its group's values and
// no bound is checked.
template <int S, int V, int K, int H>
__global__ __launch_bounds__(kTopkThreads) void topk_fixed(const float* __restrict__ logits,
                                                           int64_t n, int renorm,
                                                           int* __restrict__ idx,
                                                           float* __restrict__ wout) {
  constexpr int E = S * V;
  constexpr int EG = E / H;
  constexpr int KG = K / H;
  static_assert(E % H == 0 && K % H == 0 && EG % S == 0 && KG <= EG, "fixed top-K shape");
  const int lane = threadIdx.x & (kWave - 1);
  const int s = lane & (S - 1);
  const int seg_base = lane & ~(S - 1);
  const int64_t tok = (static_cast<int64_t>(blockIdx.x) * kTopkThreads + threadIdx.x) / S;
  const bool active = tok < n;  // inactive lanes read row 0 and still join the cross-lane steps
  const float* row = logits + (active ? tok : 0) * static_cast<int64_t>(E);

  float val[V];
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) val[v] = row[s + S * v];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = order_key(val[v]);

  float selv[K];
  int selc[K];
#pragma unroll
  for (int r = 0; r < K; ++r) {
    const int g = r / KG;
    uint32_t best = 0u;
    int bv = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if ((S * v) / EG != g) continue;  // compile-time after unrolling
      if (key[v] > best) {  // strict: lowest v on equal keys
        best = key[v];
        bv = v;
      }
    }
    const uint32_t m = seg_max<S>(best);
    int col;
    if (V == 1) {
      const uint64_t tie = __ballot(best == m);
      const uint64_t mine = (tie >> seg_base) & (S == 64 ? ~0ull : ((1ull << S) - 1));
      col = __builtin_ctzll(mine);
    } else {
      col = static_cast<int>(
          seg_min<S>(best == m ? static_cast<uint32_t>(s + S * bv) : 0xffffffffu));
    }
    // remove the pick: the winning lane (col % S) drops its best value,
    // which is the pick itself (value bv, the lowest v on equal keys)
    const bool mine = s == (col & (S - 1));
#pragma unroll
    for (int v = 0; v < V; ++v)
      if ((S * v) / EG == g) key[v] = (mine && bv == v) ? 0u : key[v];
    selc[r] = col;
    selv[r] = key_float(m);
  }

  // Lane s < K of the segment finishes pick s: its weight is one exponential
  // and one division, the softmax sum a segment reduction (over the group's
  // KG lanes when KG is a power of two, else over the whole segment, H = 1).
  static_assert(K <= S, "one lane per pick");
  static_assert(H == 1 || (KG & (KG - 1)) == 0, "groups reduce over aligned lane groups");
  float mysel = selv[0];
  int mycol = selc[0];
#pragma unroll
  for (int r = 1; r < K; ++r) {
    if (s == r) {
      mysel = selv[r];
      mycol = selc[r];
    }
  }
  const int g = s / KG;
  float w;
  if (renorm) {
    float gmax = selv[0];  // a group's first pick is its max
#pragma unroll
    for (int q = 1; q < H; ++q)
      if (g == q) gmax = selv[q * KG];
    const float e = s < K ? __expf(mysel - gmax) : 0.f;
    float z = e;
    if (H == 1) {
#pragma unroll
      for (int o = S / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, kWave);
    } else {
#pragma unroll
      for (int o = KG / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, kWave);
    }
    w = __fdividef(e, z);
  } else {
    float mall = selv[0];
#pragma unroll
    for (int q = 1; q < H; ++q) mall = fmaxf(mall, selv[q * KG]);
    float zl = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) zl += __expf(val[v] - mall);
#pragma unroll
    for (int o = S / 2; o > 0; o >>= 1) zl += __shfl_xor(zl, o, kWave);
    w = __fdividef(__expf(mysel - mall), zl);
  }
  if (active && s < K) {
    idx[tok * K + s] = mycol;
    if (wout) wout[tok * K + s] = w;
  }
}

template <int S, int V>
static void launch_topk(const float* logits, int64_t n, int E, int K, int H, int renorm,
                        int* idx, float* w, hipStream_t s) {
  const unsigned grid = ceil_div(n * S, kTopkThreads);
  topk_kernel<S, V><<<grid, kTopkThreads, 0, s>>>(logits, n, E, K, H, renorm, idx, w);
}

}  // namespace route

using namespace route;

ROUTE_API int route_topk(const float* logits, int64_t n, int32_t E, int32_t K, int32_t H,
                         int32_t renorm, int32_t* idx, float* weights, hipStream_t s) {
  if (n < 0 || E < 1 || K < 1 || H < 1 || E % H != 0 || K % H != 0 || K / H > E / H)
    return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!logits || !idx) return ROUTE_ERR_NULL;
  // shapes of the routing workloads, fixed at compile time
#define ROUTE_FIXED(s_, v_, k_, h_)                                                       \
  if (E == s_ * v_ && K == k_ && H == h_) {                                               \
    topk_fixed<s_, v_, k_, h_><<<ceil_div(n * s_, kTopkThreads), kTopkThreads, 0, s>>>(   \
        logits, n, renorm, idx, weights);                                                 \
    return launch_status();                                                               \
  }
  ROUTE_FIXED(16, 10, 6, 1)
  ROUTE_FIXED(16, 8, 8, 1)
  ROUTE_FIXED(16, 4, 8, 4)
  ROUTE_FIXED(8, 1, 2, 1)
  ROUTE_FIXED(4, 1, 2, 1)
#undef ROUTE_FIXED
  if (E <= 4)
    launch_topk<4, 1>(logits, n, E, K, H, renorm, idx, weights, s);
  else if (E <= 8)
    launch_topk<8, 1>(logits, n, E, K, H, renorm, idx, weights, s);
  else if (E <= 16)
    launch_topk<16, 1>(logits, n, E, K, H, renorm, idx, weights, s);
  else if (E <= 32)
    launch_topk<32, 1>(logits, n, E, K, H, renorm, idx, weights, s);
  else if (E <= 256) {
    switch ((E + 15) / 16) {
#define ROUTE_V16_CASE(v) \
  case v: launch_topk<16, v>(logits, n, E, K, H, renorm, idx, weights, s); break;
      ROUTE_V16_CASE(3) ROUTE_V16_CASE(4) ROUTE_V16_CASE(5) ROUTE_V16_CASE(6) ROUTE_V16_CASE(7)
      ROUTE_V16_CASE(8) ROUTE_V16_CASE(9) ROUTE_V16_CASE(10) ROUTE_V16_CASE(11)
      ROUTE_V16_CASE(12) ROUTE_V16_CASE(13) ROUTE_V16_CASE(14) ROUTE_V16_CASE(15)
      ROUTE_V16_CASE(16)
#undef ROUTE_V16_CASE
      default: return ROUTE_ERR_UNSUPPORTED;
    }
  } else {
    switch ((E + 63) / 64) {
#define ROUTE_V_CASE(v) \
  case v: launch_topk<64, v>(logits, n, E, K, H, renorm, idx, weights, s); break;
      ROUTE_V_CASE(5) ROUTE_V_CASE(6) ROUTE_V_CASE(7) ROUTE_V_CASE(8) ROUTE_V_CASE(9)
      ROUTE_V_CASE(10) ROUTE_V_CASE(11) ROUTE_V_CASE(12) ROUTE_V_CASE(13) ROUTE_V_CASE(14)
      ROUTE_V_CASE(15) ROUTE_V_CASE(16)
#undef ROUTE_V_CASE
      default: return ROUTE_ERR_UNSUPPORTED;
    }
  }
  return launch_status();
}
