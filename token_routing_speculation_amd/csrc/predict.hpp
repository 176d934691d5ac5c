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

}  // namespace route
