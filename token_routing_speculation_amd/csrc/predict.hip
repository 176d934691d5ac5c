// route_predict and route_lut_build: the lookup-table route prediction of
// "Speculative MoE" notes, section 4.1. Prediction is a table gather per
// token (intra-layer token table, 2-gram cluster table as the fallback when
// the token table's confidence is low); the builder reduces each token id's
// routing to its most-weighted cluster and a confidence byte.
#include "common.hpp"
#include "csort.hpp"
#include "predict.hpp"

namespace route {

constexpr int kPredThreads = 256;

__global__ __launch_bounds__(kPredThreads) void predict_kernel(PredictArgs a, int64_t n,
                                                              uint8_t* __restrict__ dest) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPredThreads + threadIdx.x;
  if (i >= n) return;
  const int c = predict_cluster(a, i);
  if (c >= a.G) set_err(a.err, ROUTE_EBIT_DEST_RANGE);
  dest[i] = static_cast<uint8_t>(c);
}

// The sort's key source for route_predict_sort: token j's prediction, also
// written to dest[j] (a key read again writes the same byte). A batch is
// predicted in stages (predict_stage1/2/3), each stage's loads issued for
// every key before any is used, and its error bits are flagged once.
struct PredictKeys {
  PredictArgs a;
  uint8_t* dest;
  template <int NB>
  __device__ __forceinline__ void batch(const int64_t (&j)[NB], const bool (&in)[NB],
                                        uint32_t (&k)[NB]) const {
    PredictLoads s[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) s[q] = predict_stage1(a, in[q] ? j[q] : 0);
#pragma unroll
    for (int q = 0; q < NB; ++q) predict_stage2(a, s[q]);
    uint32_t e = 0;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      uint32_t eq = 0;
      const int c = predict_stage3(a, s[q], &eq);
      if (in[q]) {
        dest[j[q]] = static_cast<uint8_t>(c);
        e |= eq;
      }
      k[q] = in[q] ? static_cast<uint32_t>(c) : 0xffffffffu;
    }
    if (e) set_err(a.err, e);
  }
};

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
  const PredictArgs a{tok, lut, conf, vocab, prev2, prev1, ngram, G, conf_thr, err};
  predict_kernel<<<ceil_div(n, kPredThreads), kPredThreads, 0, s>>>(a, n, dest);
  return launch_status();
}

ROUTE_API int route_predict_sort(const int32_t* tok, int64_t n, const uint8_t* lut,
                                 const uint8_t* conf, int32_t vocab, const uint8_t* prev2,
                                 const uint8_t* prev1, const uint8_t* ngram, int32_t G,
                                 int32_t conf_thr, uint8_t* dest, int32_t* cluster_offsets,
                                 int32_t* row_of_src, int32_t* src_of_row, uint8_t* row_cluster,
                                 void* ws, size_t ws_bytes, uint32_t* err, hipStream_t s) {
  if (n < 0 || vocab < 1 || G < 1 || n >= (int64_t(1) << 31)) return ROUTE_ERR_SHAPE;
  if (G > kMaxClusters) return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    return launch_status();
  }
  if (!tok || !lut || !dest || !row_of_src || !src_of_row) return ROUTE_ERR_NULL;
  if (conf && (!prev2 || !prev1 || !ngram)) return ROUTE_ERR_NULL;
  if (!ws || ws_bytes < csort_ws_bytes(n, G)) return ROUTE_ERR_WORKSPACE;
  const PredictKeys src{PredictArgs{tok, lut, conf, vocab, prev2, prev1, ngram, G, conf_thr, err},
                        dest};
  return csort_launch_src(src, static_cast<const uint8_t*>(dest), n, G, cluster_offsets,
                          row_of_src, src_of_row, row_cluster, ws, err, ROUTE_EBIT_DEST_RANGE, s);
}

ROUTE_API size_t route_predict_sort_workspace_size(int64_t n, int32_t G) {
  if (n < 0 || G < 1 || G > kMaxClusters) return 0;
  return csort_ws_bytes(n, G);
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
