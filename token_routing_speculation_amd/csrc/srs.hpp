// Pieces of the shuffled reduce ("Speculative MoE", section 3.1, s-TS)
// shared by its row mover (srs.hip) and by the mover fused with the router
// product (mma.hip).
#pragma once

#include "common.hpp"

namespace route {

// Outputs of a shuffle without a sort (one cluster): cluster offsets {0, n}
// and identity maps, written by the row mover itself instead of by separate
// fill launches. Each pointer may be null.
struct SrsIdentity {
  int* offsets;
  int* row_of_src;
  int* src_of_row;
  uint8_t* row_cluster;
};

// Source row i's share of the identity outputs (one thread per row).
__device__ __forceinline__ void write_identity_row(const SrsIdentity& id, int64_t i, int64_t n) {
  if (id.offsets && i == 0) {
    id.offsets[0] = 0;
    id.offsets[1] = static_cast<int>(n);
  }
  if (id.row_of_src) id.row_of_src[i] = static_cast<int>(i);
  if (id.src_of_row) id.src_of_row[i] = static_cast<int>(i);
  if (id.row_cluster) id.row_cluster[i] = 0;
}

// The router's top-K and local count taken in the fused kernel's epilogue
// (srs_shuffle_route): idx [n][K] and weights [n][K] (nullable) at the sorted
// row, *local += the picks whose expert_cluster equals the row's predicted
// cluster dest[i] (0 without dest); no count when expert_cluster is null.
struct GateTopk {
  int K;
  int renorm;
  int* idx;
  float* weights;
  const uint8_t* dest;
  const uint8_t* expert_cluster;
  unsigned long long* local;
  // grouped top-K ("Federation of Experts (FoE)" article): H groups of E / H
  // experts, each picking its K / H (H <= 1: plain top-K); the local count
  // then compares group h's picks with lar_cluster[row * H + h] (nullable:
  // dest[row], as with one group)
  int H;
  const uint8_t* lar_cluster;
};

// mma.hip: the fused shuffle + router kernel for 1 <= E <= 160 columns,
// P in {1, 2, 4} partials and d % 128 == 0 (d >= 128). out[dst(i)] =
// bf16(sum_p partials[p][i]) exactly as the row mover computes it, and
// logits[dst(i)][e] = out[dst(i)] . w[e] (binary32), dst(i) = row_of_src[i]
// (the identity when row_of_src is null; rows whose dst is out of range are
// skipped; logits may be null when topk is given). With topk (nullable) the
// epilogue also takes each row's top-K and count. Returns
// ROUTE_ERR_UNSUPPORTED for any other shape.
bool srs_gate_fits(int P, int d, int E);
int srs_gate_launch(const uint16_t* partials, int P, int64_t n, int d, const int* row_of_src,
                    uint16_t* out, const uint16_t* w, int E, float* logits,
                    const SrsIdentity& ident, const GateTopk* topk, hipStream_t s);

}  // namespace route
