// route_predict and route_lut_build: the lookup-table route prediction of
// "Speculative MoE" notes, section 4.1. Prediction is a table gather per
// token (intra-layer token table, 2-gram cluster table as the fallback when
// the token table's confidence is low); the builder reduces each token id's
// routing to its most-weighted cluster and a confidence byte.
#include "common.hpp"

namespace route {

constexpr int kPredThreads = 256;

__global__ __launch_bounds__(kPredThreads) void predict_kernel(
    const int32_t* __restrict__ tok, int64_t n, const uint8_t* __restrict__ lut,
    const uint8_t* __restrict__ conf, int vocab, const uint8_t* __restrict__ prev2,
    const uint8_t* __restrict__ prev1, const uint8_t* __restrict__ ngram, int G, int conf_thr,
    uint8_t* __restrict__ dest, uint32_t* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPredThreads + threadIdx.x;
  if (i >= n) return;
  const int t = tok[i];
  if (t < 0 || t >= vocab) {
    dest[i] = 0;
    set_err(err, ROUTE_EBIT_TOKEN_RANGE);
    return;
  }
  int c = lut[t];
  if (conf && static_cast<int>(conf[t]) < conf_thr) {
    const int a = prev2[i];
    const int b = prev1[i];
    if (a < G && b < G) {
      c = ngram[a * G + b];
    } else {
      c = 0;
      set_err(err, ROUTE_EBIT_DEST_RANGE);
    }
  }
  if (c >= G) set_err(err, ROUTE_EBIT_DEST_RANGE);
  dest[i] = static_cast<uint8_t>(c);
}

// One thread per row. The share of the cluster of slot k is recomputed as a
// binary32 sum over the slots in k order, so every cluster's share has one
// fixed summation order.
__global__ __launch_bounds__(kPredThreads) void lut_build_kernel(
    const int32_t* __restrict__ ids, int64_t n, const int32_t* __restrict__ idx,
    const float* __restrict__ w, int K, const uint8_t* __restrict__ expert_cluster, int E, int G,
    uint8_t* __restrict__ lut, uint8_t* __restrict__ conf, int vocab, uint32_t* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPredThreads + threadIdx.x;
  if (i >= n) return;
  const int id = ids[i];
  if (id < 0 || id >= vocab) {
    set_err(err, ROUTE_EBIT_TOKEN_RANGE);
    return;
  }
  int cl[kMaxK];
  float wk[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    cl[k] = -1;
    wk[k] = 0.f;
    if (k < K) {
      const int e = idx[i * K + k];
      if (e >= 0 && e < E) {
        const int c = expert_cluster[e];
        if (c < G) {
          cl[k] = c;
          wk[k] = w[i * K + k];
        } else {
          set_err(err, ROUTE_EBIT_DEST_RANGE);
        }
      } else {
        set_err(err, ROUTE_EBIT_EXPERT_RANGE);
      }
    }
  }
  auto share = [&](int c) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (cl[k] == c) s += wk[k];
    return s;
  };
  // cluster 0 is the default winner (its share is 0 when no slot sits there)
  int best_c = 0;
  float best_s = share(0);
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (cl[k] > 0) {
      const float s = share(cl[k]);
      if (s > best_s || (s == best_s && cl[k] < best_c)) {
        best_s = s;
        best_c = cl[k];
      }
    }
  }
  lut[id] = static_cast<uint8_t>(best_c);
  if (conf) {
    const float t = floorf(__fadd_rn(__fmul_rn(255.0f, best_s), 0.5f));
    conf[id] = static_cast<uint8_t>(fminf(255.f, fmaxf(0.f, t)));
  }
}

}  // namespace route

using namespace route;

ROUTE_API int route_predict(const int32_t* tok, int64_t n, const uint8_t* lut,
                            const uint8_t* conf, int32_t vocab, const uint8_t* prev2,
                            const uint8_t* prev1, const uint8_t* ngram, int32_t G,
                            int32_t conf_thr, uint8_t* dest, uint32_t* err, hipStream_t s) {
  if (n < 0 || vocab < 1 || G < 1) return ROUTE_ERR_SHAPE;
  if (G > kMaxClusters) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!tok || !lut || !dest) return ROUTE_ERR_NULL;
  if (conf && (!prev2 || !prev1 || !ngram)) return ROUTE_ERR_NULL;
  predict_kernel<<<ceil_div(n, kPredThreads), kPredThreads, 0, s>>>(
      tok, n, lut, conf, vocab, prev2, prev1, ngram, G, conf_thr, dest, err);
  return launch_status();
}

ROUTE_API int route_lut_build(const int32_t* ids, int64_t n, const int32_t* idx, const float* w,
                              int32_t K, const uint8_t* expert_cluster, int32_t E, int32_t G,
                              uint8_t* lut, uint8_t* conf, int32_t vocab, uint32_t* err,
                              hipStream_t s) {
  if (n < 0 || K < 1 || E < 1 || G < 1 || vocab < 1) return ROUTE_ERR_SHAPE;
  if (G > kMaxClusters || K > kMaxK || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!ids || !idx || !w || !expert_cluster || !lut) return ROUTE_ERR_NULL;
  lut_build_kernel<<<ceil_div(n, kPredThreads), kPredThreads, 0, s>>>(
      ids, n, idx, w, K, expert_cluster, E, G, lut, conf, vocab, err);
  return launch_status();
}
