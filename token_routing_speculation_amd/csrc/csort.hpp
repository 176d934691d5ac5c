// Stable counting sort of small integer keys, in three launches:
//   1. csort_hist:  per-chunk histograms in LDS, written bin-major [B][nchunks];
//   2. csort_scan:  one workgroup scans the bin-major table (exclusive), so
//                   base[b][c] is where chunk c's first key of bin b lands, and
//                   writes the bin offsets [B+1];
//   3. csort_rank:  per chunk, keys are ranked in order (256 at a time) with a
//                   ballot-based match of equal keys inside each wave, a prefix
//                   over the block's waves and a running per-bin count, giving
//                   each key its stable position.
// Keys >= B (or negative) are skipped: flagged in err, position -1.
#pragma once

#include "common.hpp"

namespace route {
namespace {  // internal linkage: each translation unit gets its own copy

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kScanThreads = 1024;
constexpr int kMaxScanEntries = 65536;

// Keys per chunk: 1024, doubled until the bin-major table fits one scan block.
inline int64_t csort_chunk(int64_t n, int B) {
  int64_t chunk = 1024;
  while (static_cast<int64_t>(B) * ((n + chunk - 1) / chunk) > kMaxScanEntries) chunk *= 2;
  return chunk;
}

inline int64_t csort_nchunks(int64_t n, int B) {
  int64_t c = csort_chunk(n, B);
  return n == 0 ? 0 : (n + c - 1) / c;
}

// Bytes of scratch: hist and base tables, 256-byte aligned each.
inline size_t csort_ws_bytes(int64_t n, int B) {
  size_t t = static_cast<size_t>(B) * static_cast<size_t>(csort_nchunks(n, B)) * sizeof(int);
  return 2 * align_up(t, 256);
}

template <typename KeyT>
__device__ __forceinline__ uint32_t key_u32(KeyT k) {
  return static_cast<uint32_t>(k);
}
template <>
__device__ __forceinline__ uint32_t key_u32<int32_t>(int32_t k) {
  return k < 0 ? 0xffffffffu : static_cast<uint32_t>(k);
}

template <typename KeyT>
__global__ __launch_bounds__(kSortThreads) void csort_hist(const KeyT* __restrict__ keys,
                                                           int64_t n, int B, int64_t chunk,
                                                           int nchunks, int* __restrict__ hist,
                                                           uint32_t* err, uint32_t ebit) {
  __shared__ int h[kMaxExperts];
  for (int b = threadIdx.x; b < B; b += kSortThreads) h[b] = 0;
  __syncthreads();
  const int64_t c = blockIdx.x;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  bool bad = false;
  for (int64_t j = lo + threadIdx.x; j < hi; j += kSortThreads) {
    uint32_t k = key_u32<KeyT>(keys[j]);
    if (k < static_cast<uint32_t>(B))
      atomicAdd(&h[k], 1);
    else
      bad = true;
  }
  if (bad) set_err(err, ebit);
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += kSortThreads)
    hist[static_cast<int64_t>(b) * nchunks + c] = h[b];
}

// Exclusive scan of the bin-major table (M = B * nchunks entries) by one
// workgroup; also writes offsets[b] = first slot of bin b, offsets[B] = total.
__global__ __launch_bounds__(kScanThreads) void csort_scan(const int* __restrict__ hist, int M,
                                                           int B, int nchunks,
                                                           int* __restrict__ base,
                                                           int* __restrict__ offsets) {
  __shared__ int part[kScanThreads];
  const int t = threadIdx.x;
  const int per = (M + kScanThreads - 1) / kScanThreads;
  const int lo = t * per;
  const int hi = lo + per < M ? lo + per : M;
  int s = 0;
  for (int j = lo; j < hi; ++j) s += hist[j];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int o = 1; o < kScanThreads; o <<= 1) {
    int v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t == 0 ? 0 : part[t - 1];
  for (int j = lo; j < hi; ++j) {
    base[j] = run;
    if (nchunks > 0 && j % nchunks == 0) offsets[j / nchunks] = run;
    run += hist[j];
  }
  if (t == kScanThreads - 1) offsets[B] = part[kScanThreads - 1];
}

// Ranks the keys of chunk blockIdx.x. fwd[j] = position of key j,
// inv[pos] = j, inv_key[pos] = key (inv_key nullable).
template <typename KeyT>
__global__ __launch_bounds__(kSortThreads) void csort_rank(const KeyT* __restrict__ keys,
                                                           int64_t n, int B, int nbits,
                                                           int64_t chunk, int nchunks,
                                                           const int* __restrict__ base,
                                                           int* __restrict__ fwd,
                                                           int* __restrict__ inv,
                                                           uint8_t* __restrict__ inv_key) {
  __shared__ int sbase[kMaxExperts];
  __shared__ int srun[kMaxExperts];
  __shared__ int wcnt[kSortWaves][kMaxExperts];
  const int t = threadIdx.x;
  const int w = t / kWave;
  const int lane = t & (kWave - 1);
  const int64_t c = blockIdx.x;
  for (int b = t; b < B; b += kSortThreads) {
    sbase[b] = base[static_cast<int64_t>(b) * nchunks + c];
    srun[b] = 0;
#pragma unroll
    for (int v = 0; v < kSortWaves; ++v) wcnt[v][b] = 0;
  }
  __syncthreads();
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t j0 = lo; j0 < hi; j0 += kSortThreads) {
    const int64_t j = j0 + t;
    uint32_t k = 0xffffffffu;
    if (j < hi) k = key_u32<KeyT>(keys[j]);
    const bool valid = k < static_cast<uint32_t>(B);
    // lanes of this wave holding the same valid key
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((k >> bit) & 1u);
      const uint64_t bs = __ballot(set);
      m &= set ? bs : ~bs;
    }
    const int rank = __popcll(m & below);
    const int total = __popcll(m);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[w][k] = total;
    __syncthreads();
    if (valid) {
      int pre = 0;
#pragma unroll
      for (int v = 0; v < kSortWaves; ++v) pre += v < w ? wcnt[v][k] : 0;
      const int pos = sbase[k] + srun[k] + pre + rank;
      fwd[j] = pos;
      inv[pos] = static_cast<int>(j);
      if (inv_key) inv_key[pos] = static_cast<uint8_t>(k);
    } else if (j < hi) {
      fwd[j] = -1;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&srun[k], total);
      wcnt[w][k] = 0;
    }
    __syncthreads();
  }
}

__global__ void fill_i32(int* __restrict__ p, int64_t n, int value) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

__global__ void iota_i32(int* __restrict__ p, int64_t n) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = static_cast<int>(i);
}

__global__ void fill_u8(uint8_t* __restrict__ p, int64_t n, uint8_t value) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

inline int bits_for(int B) {
  int nb = 0;
  while ((1 << nb) < B) ++nb;
  return nb;
}

// Enqueues the three sort launches. ws holds the two tables.
template <typename KeyT>
int csort_launch(const KeyT* keys, int64_t n, int B, int* offsets, int* fwd, int* inv,
                 uint8_t* inv_key, void* ws, uint32_t* err, uint32_t ebit, hipStream_t s) {
  if (n == 0) {
    fill_i32<<<ceil_div(B + 1, 256), 256, 0, s>>>(offsets, B + 1, 0);
    return launch_status();
  }
  const int64_t chunk = csort_chunk(n, B);
  const int nch = static_cast<int>(csort_nchunks(n, B));
  const size_t t = align_up(static_cast<size_t>(B) * nch * sizeof(int), 256);
  int* hist = static_cast<int*>(ws);
  int* base = reinterpret_cast<int*>(static_cast<char*>(ws) + t);
  csort_hist<KeyT><<<nch, kSortThreads, 0, s>>>(keys, n, B, chunk, nch, hist, err, ebit);
  csort_scan<<<1, kScanThreads, 0, s>>>(hist, B * nch, B, nch, base, offsets);
  csort_rank<KeyT><<<nch, kSortThreads, 0, s>>>(keys, n, B, bits_for(B), chunk, nch, base, fwd,
                                                 inv, inv_key);
  return launch_status();
}

}  // namespace
}  // namespace route
