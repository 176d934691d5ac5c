// srs_shuffle: the shuffled reduce-scatter of "Speculative MoE" (section 3.1,
// s-TS) on one GPU. The P tensor-parallel partials of each token are summed
// in binary32 (partial order 0..P-1) and rounded once to bf16, and the row is
// written straight into its predicted cluster's contiguous row range, so the
// reduce and the shuffle are one pass over HBM: P rows read, one row written.
//
// The destination row of every token comes from a stable counting sort of
// the uint8 cluster ids (csort.hpp); the row mover then streams each source
// row with 16-byte vector loads, one wave per row. srs_shuffle_gate runs the
// same sort, then the reduce fused with the router product on its output
// (mma.hip), so the reduced rows are multiplied before they leave the chip.
#include "common.hpp"
#include "csort.hpp"
#include "srs.hpp"

namespace route {

constexpr int kMoveThreads = 256;

// row i's share of the identity outputs (lane 0 of row i's wave)
__device__ __forceinline__ void write_identity(const SrsIdentity& id, int64_t i, int64_t n) {
  if (lane_id() == 0) write_identity_row(id, i, n);
}

// One wave per source row: out[dst(i)] = bf16(sum_p partials[p][i]). Every
// lane first loads all P x CPL of its 16-byte vectors, then sums and stores.
// Cache policy, measured on MI355X for this pattern: streaming (nontemporal)
// loads with plain stores move about 6.5 TB/s, against 5.4 TB/s with both
// streaming.
template <int PT, int CPL>
__global__ __launch_bounds__(kMoveThreads) void srs_move(const uint16_t* __restrict__ partials,
                                                         int64_t n, int d,
                                                         const int* __restrict__ row_of_src,
                                                         uint16_t* __restrict__ out,
                                                         SrsIdentity ident) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kMoveThreads / kWave) + wave_id();
  if (i >= n) return;
  write_identity(ident, i, n);
  const int dst = row_of_src ? row_of_src[i] : static_cast<int>(i);
  if (dst < 0 || dst >= n) return;
  const int lane = lane_id();
  const int nv = d >> 3;  // 16-byte vectors per row
  const size_t plane = static_cast<size_t>(n) * d;
  const uint16_t* src = partials + static_cast<size_t>(i) * d;
  uint16_t* o = out + static_cast<size_t>(dst) * d;
  // vectors past the row end load vector 0 again (in bounds) and are never stored
  u32x4 x[PT][CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    const int vv = v < nv ? v : 0;
#pragma unroll
    for (int p = 0; p < PT; ++p) x[p][c] = ld16_stream(src + p * plane + 8 * vv);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int v = lane + c * kWave;
    float acc[8];
    unpack8(x[0][c], acc);
#pragma unroll
    for (int p = 1; p < PT; ++p) {
      float f[8];
      unpack8(x[p][c], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += f[e];
    }
    if (v < nv) st16(o + 8 * v, pack8_cvt(acc));
  }
}

// Any P and row length: a plain loop over the row, partial by partial.
__global__ __launch_bounds__(kMoveThreads) void srs_move_any(const uint16_t* __restrict__ partials,
                                                             int P, int64_t n, int d,
                                                             const int* __restrict__ row_of_src,
                                                             uint16_t* __restrict__ out,
                                                             SrsIdentity ident) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kMoveThreads / kWave) + wave_id();
  if (i >= n) return;
  write_identity(ident, i, n);
  const int dst = row_of_src ? row_of_src[i] : static_cast<int>(i);
  if (dst < 0 || dst >= n) return;
  const int nv = d >> 3;
  const size_t plane = static_cast<size_t>(n) * d;
  const uint16_t* src = partials + static_cast<size_t>(i) * d;
  uint16_t* o = out + static_cast<size_t>(dst) * d;
  for (int v = lane_id(); v < nv; v += kWave) {
    float acc[8];
    unpack8(ld16_stream(src + 8 * v), acc);
    for (int p = 1; p < P; ++p) {
      float f[8];
      unpack8(ld16_stream(src + p * plane + 8 * v), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += f[e];
    }
    st16(o + 8 * v, pack8_cvt(acc));
  }
}

// vectors per lane for a row of nv 16-byte vectors (0: no instantiated size)
static int srs_cpl(int nv) {
  const int need = (nv + kWave - 1) / kWave;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 10 ? 10 : 0;
}

template <int PT>
static bool launch_srs_move(int cpl, unsigned grid, hipStream_t s, const uint16_t* partials,
                            int64_t n, int d, const int* fwd, uint16_t* out,
                            const SrsIdentity& ident) {
  switch (cpl) {
#define ROUTE_SRS_CASE(c)                                                                   \
  case c:                                                                                   \
    srs_move<PT, c><<<grid, kMoveThreads, 0, s>>>(partials, n, d, fwd, out, ident);         \
    return true;
    ROUTE_SRS_CASE(1) ROUTE_SRS_CASE(2) ROUTE_SRS_CASE(4) ROUTE_SRS_CASE(8) ROUTE_SRS_CASE(10)
#undef ROUTE_SRS_CASE
    default: return false;
  }
}

static size_t srs_ws(int64_t n, int G) {
  return csort_ws_bytes(n, G) + align_up(static_cast<size_t>(n) * sizeof(int), 256) +
         align_up(static_cast<size_t>(n) * sizeof(int), 256);
}

}  // namespace route

using namespace route;

ROUTE_API size_t srs_shuffle_workspace_size(int64_t n, int32_t G) {
  if (n < 0 || G < 1 || G > kMaxClusters) return 0;
  return srs_ws(n, G);
}

ROUTE_API int srs_shuffle(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                          const uint8_t* dest, int32_t G, uint16_t* out,
                          int32_t* cluster_offsets, int32_t* row_of_src, int32_t* src_of_row,
                          uint8_t* row_cluster, void* ws, size_t ws_bytes, uint32_t* err,
                          hipStream_t s) {
  if (n < 0 || P < 1 || d < 8 || d % 8 != 0 || G < 1 || n >= (int64_t(1) << 31))
    return ROUTE_ERR_SHAPE;
  if (P > 16 || G > kMaxClusters) return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    return launch_status();
  }
  if (!partials || !out) return ROUTE_ERR_NULL;
  if (!dest && G != 1) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(out)) return ROUTE_ERR_ALIGN;
  const bool sort = dest != nullptr;
  if (sort) {
    if (!ws) return ROUTE_ERR_WORKSPACE;
    if (ws_bytes < srs_ws(n, G)) return ROUTE_ERR_WORKSPACE;
  }
  const int* fwd = nullptr;
  if (sort) {
    char* w = static_cast<char*>(ws);
    const size_t ct = csort_ws_bytes(n, G);
    const size_t nt = align_up(static_cast<size_t>(n) * sizeof(int), 256);
    int* fwd_buf = row_of_src ? row_of_src : reinterpret_cast<int*>(w + ct);
    int* inv_buf = src_of_row ? src_of_row : reinterpret_cast<int*>(w + ct + nt);
    int st = csort_launch<uint8_t>(dest, n, G, cluster_offsets, fwd_buf, inv_buf, row_cluster,
                                   w, err, ROUTE_EBIT_DEST_RANGE, s);
    if (st != ROUTE_OK) return st;
    fwd = fwd_buf;
  }
  // single cluster, no shuffle: the mover writes offsets {0, n} and identity maps
  const SrsIdentity ident = sort ? SrsIdentity{nullptr, nullptr, nullptr, nullptr}
                                 : SrsIdentity{cluster_offsets, row_of_src, src_of_row, row_cluster};
  const unsigned grid = ceil_div(n, kMoveThreads / kWave);
  const int cpl = srs_cpl(d / 8);
  bool done = false;
  if (P == 1) done = launch_srs_move<1>(cpl, grid, s, partials, n, d, fwd, out, ident);
  if (P == 2) done = launch_srs_move<2>(cpl, grid, s, partials, n, d, fwd, out, ident);
  if (P == 4 && cpl <= 4) done = launch_srs_move<4>(cpl, grid, s, partials, n, d, fwd, out, ident);
  if (!done) srs_move_any<<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out, ident);
  return launch_status();
}

ROUTE_API int srs_shuffle_gate(const uint16_t* partials, int32_t P, int64_t n, int32_t d,
                               const uint8_t* dest, int32_t G, uint16_t* out,
                               int32_t* cluster_offsets, int32_t* row_of_src,
                               int32_t* src_of_row, uint8_t* row_cluster, const uint16_t* w,
                               int32_t E, float* logits, void* ws, size_t ws_bytes,
                               uint32_t* err, hipStream_t s) {
  if (n < 0 || P < 1 || d < 8 || d % 8 != 0 || G < 1 || E < 1 || n >= (int64_t(1) << 31))
    return ROUTE_ERR_SHAPE;
  if (G > kMaxClusters || !srs_gate_fits(P, d, E)) return ROUTE_ERR_UNSUPPORTED;
  if (!cluster_offsets) return ROUTE_ERR_NULL;
  if (n == 0) {
    fill_i32<<<ceil_div(G + 1, 256), 256, 0, s>>>(cluster_offsets, G + 1, 0);
    return launch_status();
  }
  if (!partials || !out || !w || !logits) return ROUTE_ERR_NULL;
  if (!dest && G != 1) return ROUTE_ERR_NULL;
  if (!aligned16(partials) || !aligned16(out) || !aligned16(w)) return ROUTE_ERR_ALIGN;
  const bool sort = dest != nullptr;
  if (sort) {
    if (!ws) return ROUTE_ERR_WORKSPACE;
    if (ws_bytes < srs_ws(n, G)) return ROUTE_ERR_WORKSPACE;
  }
  const int* fwd = nullptr;
  if (sort) {
    char* wsp = static_cast<char*>(ws);
    const size_t ct = csort_ws_bytes(n, G);
    const size_t nt = align_up(static_cast<size_t>(n) * sizeof(int), 256);
    int* fwd_buf = row_of_src ? row_of_src : reinterpret_cast<int*>(wsp + ct);
    int* inv_buf = src_of_row ? src_of_row : reinterpret_cast<int*>(wsp + ct + nt);
    int st = csort_launch<uint8_t>(dest, n, G, cluster_offsets, fwd_buf, inv_buf, row_cluster,
                                   wsp, err, ROUTE_EBIT_DEST_RANGE, s);
    if (st != ROUTE_OK) return st;
    fwd = fwd_buf;
  }
  const SrsIdentity ident = sort ? SrsIdentity{nullptr, nullptr, nullptr, nullptr}
                                 : SrsIdentity{cluster_offsets, row_of_src, src_of_row, row_cluster};
  return srs_gate_launch(partials, P, n, d, fwd, out, w, E, logits, ident, nullptr, s);
}
