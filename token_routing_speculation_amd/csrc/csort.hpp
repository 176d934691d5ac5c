// Stable counting sort of small integer keys, in two launches:
//   1. csort_hist:  per-chunk histograms in LDS, written chunk-major
//                   [nchunks][B] (at most 128 chunks);
//   2. csort_rank:  each chunk's block derives where its keys of each bin
//                   start (all earlier bins, plus this bin's count in earlier
//                   chunks), summing the table over all of its threads;
//                   block 0 also writes the bin offsets [B+1]. Each wave
//                   then ranks a contiguous share of the chunk (ballot-
//                   matched equal keys, wave-private running counts), giving
//                   each key its stable position.
// Keys >= B (or negative) are skipped: flagged in err, position -1.
#pragma once

#include "common.hpp"

namespace route {
namespace {  // internal linkage: each translation unit gets its own copy

constexpr int kSortThreads = 256;
constexpr int kMaxChunks = 128;
constexpr int kBatch = 8;  // keys (tiles) per thread loaded ahead of use

// Keys per chunk: a power of two >= 1024 giving at most kMaxChunks chunks.
inline int64_t csort_chunk(int64_t n, int B) {
  (void)B;
  int64_t chunk = 1024;
  while ((n + chunk - 1) / chunk > kMaxChunks) chunk *= 2;
  return chunk;
}

inline int64_t csort_nchunks(int64_t n, int B) {
  int64_t c = csort_chunk(n, B);
  return n == 0 ? 0 : (n + c - 1) / c;
}

// Bytes of scratch: the chunk-major histogram table, 256-byte aligned.
inline size_t csort_ws_bytes(int64_t n, int B) {
  size_t t = static_cast<size_t>(B) * static_cast<size_t>(csort_nchunks(n, B)) * sizeof(int);
  return align_up(t, 256);
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
  // keys are loaded kBatch at a time before any is counted, so the loads
  // overlap instead of each waiting behind the previous count
  for (int64_t j0 = lo + threadIdx.x; j0 < hi; j0 += kBatch * kSortThreads) {
    uint32_t k[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t j = j0 + q * kSortThreads;
      k[q] = j < hi ? key_u32<KeyT>(keys[j]) : 0xffffffffu;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (k[q] < static_cast<uint32_t>(B))
        atomicAdd(&h[k[q]], 1);
      else if (j0 + q * kSortThreads < hi)
        bad = true;
    }
  }
  if (bad) set_err(err, ebit);
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += kSortThreads) hist[c * B + b] = h[b];
}

// Lanes of this wave holding the same valid key as this lane (match by
// ballots over the key bits), and this lane's rank among them.
__device__ __forceinline__ uint64_t match_key(uint32_t k, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = valid && ((k >> bit) & 1u);
    const uint64_t bs = __ballot(set);
    m &= set ? bs : ~bs;
  }
  return m;
}

// Ranks the keys of chunk blockIdx.x. fwd[j] = position of key j,
// inv[pos] = j, inv_key[pos] = key (inv_key nullable). THREADS / 64 waves.
//
// Prologue: per bin, the total count and the count in earlier chunks. The
// threads form R = min(THREADS / B, nchunks) groups of B; group r sums chunks
// r, r + R, ... so the loads spread over all threads, and the R partial sums
// meet in LDS.
//
// The chunk is split into NW contiguous shares, one per wave. Pass 1: each
// wave counts its share per bin into its own LDS row (per 64-key tile, the
// lowest lane of each key's match adds the match size). After one barrier the
// rows become per-wave starting positions (the chunk's base for the bin plus
// the counts of the earlier shares). Pass 2: each wave walks its share again
// in order; a key's position is its wave's running start for the bin plus its
// rank among equal keys in the tile, then the lowest lane advances the start.
// Waves touch only their own LDS row, in program order, so pass 2 needs no
// barriers. More waves make each wave's serial walk shorter: the kernel is
// bound by that walk's latency, not by throughput.
template <typename KeyT, int THREADS>
__global__ __launch_bounds__(THREADS) void csort_rank(const KeyT* __restrict__ keys, int64_t n,
                                                      int B, int nbits, int64_t chunk,
                                                      int nchunks, const int* __restrict__ hist,
                                                      int* __restrict__ offsets,
                                                      int* __restrict__ fwd,
                                                      int* __restrict__ inv,
                                                      uint8_t* __restrict__ inv_key) {
  constexpr int NW = THREADS / kWave;
  // one LDS row of B counters per wave: the launch uses sixteen waves only for
  // B <= kMaxExperts / 4, and four waves for any B <= kMaxExperts
  constexpr int kMaxB = NW > 4 ? kMaxExperts / 4 : kMaxExperts;
  constexpr int kRowInts = NW * kMaxB;
  static_assert(NW == 4 || NW == 16, "launched with 256 or 1024 threads");
  __shared__ int sbase[kMaxExperts];
  __shared__ int stot[kMaxExperts];
  __shared__ int wrow[kRowInts];
  __shared__ int ppre[THREADS > kMaxExperts ? THREADS : kMaxExperts];  // R * B entries
  __shared__ int ptot[THREADS > kMaxExperts ? THREADS : kMaxExperts];
  __shared__ int stotal;
  const int t = threadIdx.x;
  const int w = wave_id();
  const int lane = t & (kWave - 1);
  const int c = blockIdx.x;
  for (int i = t; i < NW * B; i += THREADS) wrow[i] = 0;

  const int R = THREADS / B < nchunks ? (THREADS / B > 0 ? THREADS / B : 1) : nchunks;
  for (int i = t; i < R * B; i += THREADS) {  // one pass when B <= THREADS
    const int r = i / B, b = i - r * B;
    int tot = 0, pre = 0;
#pragma unroll 4
    for (int q = r; q < nchunks; q += R) {
      const int v = hist[q * B + b];
      tot += v;
      pre += q < c ? v : 0;
    }
    ppre[i] = pre;
    ptot[i] = tot;
  }
  __syncthreads();
  for (int b = t; b < B; b += THREADS) {
    int tot = 0, pre = 0;
    for (int r = 0; r < R; ++r) {
      tot += ptot[r * B + b];
      pre += ppre[r * B + b];
    }
    sbase[b] = pre;
    stot[b] = tot;
  }
  __syncthreads();
  // exclusive scan of the bin totals by wave 0 (each lane a contiguous run)
  if (w == 0) {
    const int per = (B + kWave - 1) / kWave;
    const int lo = lane * per;
    const int hi = lo + per < B ? lo + per : B;
    int local = 0;
    for (int b = lo; b < hi; ++b) local += stot[b];
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    int run = incl - local;
    for (int b = lo; b < hi; ++b) {
      const int v = stot[b];
      stot[b] = run;
      run += v;
    }
    if (lane == kWave - 1) stotal = incl;
  }
  __syncthreads();
  for (int b = t; b < B; b += THREADS) {
    if (c == 0) offsets[b] = stot[b];
    sbase[b] += stot[b];
  }
  if (c == 0 && t == 0) offsets[B] = stotal;

  // this wave's share of the chunk
  const int64_t clo = static_cast<int64_t>(c) * chunk;
  const int64_t chi = clo + chunk < n ? clo + chunk : n;
  const int64_t share = chunk / NW;
  const int64_t qlo = clo + w * share;
  const int64_t qhi = qlo + share < chi ? qlo + share : chi;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* myrow = wrow + w * B;

  // keys are read kBatch tiles (of 64) at a time, all loads issued before
  // any tile is processed; the first batch stays in registers for pass 2
  auto load_batch = [&](uint32_t (&kb)[kBatch], int64_t base) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t j = base + q * kWave + lane;
      kb[q] = j < qhi ? key_u32<KeyT>(keys[j]) : 0xffffffffu;
    }
  };
  constexpr int64_t kSpan = static_cast<int64_t>(kBatch) * kWave;
  uint32_t first[kBatch];
  load_batch(first, qlo);

  // pass 1: per-bin counts of the share
  for (int64_t jb = qlo; jb < qhi; jb += kSpan) {
    uint32_t kb[kBatch];
    if (jb == qlo) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) kb[q] = first[q];
    } else {
      load_batch(kb, jb);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (jb + q * kWave >= qhi) break;
      const uint32_t k = kb[q];
      const bool valid = k < static_cast<uint32_t>(B);
      const uint64_t m = match_key(k, valid, nbits);
      if (valid && __popcll(m & below) == 0) myrow[k] += __popcll(m);
    }
  }
  __syncthreads();
  // counts -> per-wave starting positions
  for (int b = t; b < B; b += THREADS) {
    int run = sbase[b];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int cnt = wrow[v * B + b];
      wrow[v * B + b] = run;
      run += cnt;
    }
  }
  __syncthreads();
  // pass 2: positions
  for (int64_t jb = qlo; jb < qhi; jb += kSpan) {
    uint32_t kb[kBatch];
    if (jb == qlo) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) kb[q] = first[q];
    } else {
      load_batch(kb, jb);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t j0 = jb + q * kWave;
      if (j0 >= qhi) break;
      const int64_t j = j0 + lane;
      const uint32_t k = kb[q];
      const bool valid = k < static_cast<uint32_t>(B);
      const uint64_t m = match_key(k, valid, nbits);
      const int rank = __popcll(m & below);
      int start = 0;
      if (valid) start = myrow[k];
      if (valid) {
        const int pos = start + rank;
        fwd[j] = pos;
        inv[pos] = static_cast<int>(j);
        if (inv_key) inv_key[pos] = static_cast<uint8_t>(k);
      } else if (j < qhi) {
        fwd[j] = -1;
      }
      if (valid && rank == 0) myrow[k] = start + __popcll(m);
    }
  }
}

__global__ void fill_i32(int* __restrict__ p, int64_t n, int value) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

inline int bits_for(int B) {
  int nb = 0;
  while ((1 << nb) < B) ++nb;
  return nb;
}

// Enqueues the two sort launches. ws holds the histogram table.
template <typename KeyT>
int csort_launch(const KeyT* keys, int64_t n, int B, int* offsets, int* fwd, int* inv,
                 uint8_t* inv_key, void* ws, uint32_t* err, uint32_t ebit, hipStream_t s) {
  if (n == 0) {
    fill_i32<<<ceil_div(B + 1, 256), 256, 0, s>>>(offsets, B + 1, 0);
    return launch_status();
  }
  const int64_t chunk = csort_chunk(n, B);
  const int nch = static_cast<int>(csort_nchunks(n, B));
  int* hist = static_cast<int*>(ws);
  csort_hist<KeyT><<<nch, kSortThreads, 0, s>>>(keys, n, B, chunk, nch, hist, err, ebit);
  // sixteen waves per chunk where their LDS rows fit (B <= 256), else four
  if (B <= kMaxExperts / 4)
    csort_rank<KeyT, 1024><<<nch, 1024, 0, s>>>(keys, n, B, bits_for(B), chunk, nch, hist,
                                                 offsets, fwd, inv, inv_key);
  else
    csort_rank<KeyT, kSortThreads><<<nch, kSortThreads, 0, s>>>(keys, n, B, bits_for(B), chunk,
                                                                nch, hist, offsets, fwd, inv,
                                                                inv_key);
  return launch_status();
}

}  // namespace
}  // namespace route
