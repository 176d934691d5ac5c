// srs_shuffle: the shuffled reduce-scatter of "Speculative MoE" (section 3.1,
// s-TS) on one GPU. The P tensor-parallel partials of each token are summed
// in binary32 (partial order 0..P-1) and rounded once to bf16, and the row is
// written straight into its predicted cluster's contiguous row range, so the
// reduce and the shuffle are one pass over HBM: P rows read, one row written.
//
// The destination row of every token comes from a stable counting sort of
// the uint8 cluster ids (csort.hpp); the row mover then streams each source
// row with 16-byte vector loads, one wave per row.
#include "common.hpp"
#include "csort.hpp"

namespace route {

constexpr int kMoveThreads = 256;

// One wave per source row: out[dst(i)] = bf16(sum_p partials[p][i]).
template <int PT>
__global__ __launch_bounds__(kMoveThreads) void srs_move(const uint16_t* __restrict__ partials,
                                                         int P_dyn, int64_t n, int d,
                                                         const int* __restrict__ row_of_src,
                                                         uint16_t* __restrict__ out) {
  const int P = PT > 0 ? PT : P_dyn;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kMoveThreads / kWave) + threadIdx.x / kWave;
  if (i >= n) return;
  const int dst = row_of_src ? row_of_src[i] : static_cast<int>(i);
  if (dst < 0 || dst >= n) return;
  const int lane = lane_id();
  const int nv = d >> 3;  // 16-byte vectors per row
  const size_t plane = static_cast<size_t>(n) * d;
  const uint16_t* src = partials + static_cast<size_t>(i) * d;
  uint16_t* o = out + static_cast<size_t>(dst) * d;
#pragma unroll 2
  for (int v = lane; v < nv; v += kWave) {
    float acc[8];
    unpack8(ld16_stream(src + 8 * v), acc);
    if (PT > 0) {
#pragma unroll
      for (int p = 1; p < PT; ++p) {
        float f[8];
        unpack8(ld16_stream(src + p * plane + 8 * v), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f[e];
      }
    } else {
      for (int p = 1; p < P; ++p) {
        float f[8];
        unpack8(ld16_stream(src + p * plane + 8 * v), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f[e];
      }
    }
    st16_stream(o + 8 * v, pack8(acc));
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
  } else {
    // single cluster, no shuffle: identity maps
    int* offs = cluster_offsets;
    fill_i32<<<1, 64, 0, s>>>(offs, 1, 0);
    fill_i32<<<1, 64, 0, s>>>(offs + 1, 1, static_cast<int>(n));
    if (row_of_src) iota_i32<<<ceil_div(n, 256), 256, 0, s>>>(row_of_src, n);
    if (src_of_row) iota_i32<<<ceil_div(n, 256), 256, 0, s>>>(src_of_row, n);
    if (row_cluster) fill_u8<<<ceil_div(n, 256), 256, 0, s>>>(row_cluster, n, 0);
  }
  const unsigned grid = ceil_div(n, kMoveThreads / kWave);
  switch (P) {
    case 1: srs_move<1><<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out); break;
    case 2: srs_move<2><<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out); break;
    case 3: srs_move<3><<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out); break;
    case 4: srs_move<4><<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out); break;
    default: srs_move<0><<<grid, kMoveThreads, 0, s>>>(partials, P, n, d, fwd, out); break;
  }
  return launch_status();
}
