// The route prediction of one token ("Speculative MoE" notes, section 4.1),
// shared by route_predict's kernel and the sort that route_predict_sort runs
// on the predictions as they are made.
#pragma once

#include "common.hpp"

namespace route {

// Token i's cluster: lut[tok[i]], or the 2-gram table's entry for the two
// previous layers' clusters when the fallback is on (conf given) and the
// token's confidence byte is below conf_thr. Out-of-range token: 0, flagged
// TOKEN_RANGE; previous clusters out of range: 0, flagged DEST_RANGE. The
// result may be >= G (a table entry out of range); the caller flags that.
struct PredictArgs {
  const int32_t* tok;
  const uint8_t* lut;
  const uint8_t* conf;
  int vocab;
  const uint8_t* prev2;
  const uint8_t* prev1;
  const uint8_t* ngram;
  int G;
  int conf_thr;
  uint32_t* err;
};

__device__ __forceinline__ int predict_cluster(const PredictArgs& a, int64_t i) {
  const int t = a.tok[i];
  if (t < 0 || t >= a.vocab) {
    set_err(a.err, ROUTE_EBIT_TOKEN_RANGE);
    return 0;
  }
  int c = a.lut[t];
  if (a.conf && static_cast<int>(a.conf[t]) < a.conf_thr) {
    const int p2 = a.prev2[i];
    const int p1 = a.prev1[i];
    if (p2 < a.G && p1 < a.G) {
      c = a.ngram[p2 * a.G + p1];
    } else {
      c = 0;
      set_err(a.err, ROUTE_EBIT_DEST_RANGE);
    }
  }
  return c;
}

// The same prediction in three stages with no branch around a load, for
// callers that predict a batch at once (every stage's loads issued for the
// whole batch before any is used). Stage 1 loads the token and the previous
// clusters, stage 2 the table entries (at token 0 and 2-gram entry 0 in place
// of out-of-range ones), stage 3 chooses and returns the cluster, with the
// error bits that predict_cluster would flag put in *e.
struct PredictLoads {
  int t, p2, p1, c, cf, g;
};

// (Without the fallback the previous clusters, the confidence byte and the
// 2-gram entry are read from the token table's first byte instead, so that
// no load sits under a branch; stage 3 does not use them then.)
__device__ __forceinline__ PredictLoads predict_stage1(const PredictArgs& a, int64_t i) {
  const bool fb = a.conf != nullptr;
  PredictLoads s{};
  s.t = a.tok[i];
  s.p2 = (fb ? a.prev2 : a.lut)[fb ? i : 0];
  s.p1 = (fb ? a.prev1 : a.lut)[fb ? i : 0];
  return s;
}

__device__ __forceinline__ void predict_stage2(const PredictArgs& a, PredictLoads& s) {
  const bool fb = a.conf != nullptr;
  const int tc = (s.t >= 0 && s.t < a.vocab) ? s.t : 0;
  s.c = a.lut[tc];
  s.cf = (fb ? a.conf : a.lut)[fb ? tc : 0];
  s.g = (fb ? a.ngram : a.lut)[fb && s.p2 < a.G && s.p1 < a.G ? s.p2 * a.G + s.p1 : 0];
}

__device__ __forceinline__ int predict_stage3(const PredictArgs& a, const PredictLoads& s,
                                              uint32_t* e) {
  if (s.t < 0 || s.t >= a.vocab) {
    *e |= ROUTE_EBIT_TOKEN_RANGE;
    return 0;
  }
  if (a.conf && s.cf < a.conf_thr) {
    if (s.p2 < a.G && s.p1 < a.G) return s.g;
    *e |= ROUTE_EBIT_DEST_RANGE;
    return 0;
  }
  return s.c;
}

}  // namespace route
