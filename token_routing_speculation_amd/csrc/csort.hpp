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
// Up to kSortOneMax keys the two become one launch (csort_one): a single
// workgroup counts, scans and ranks the whole array.
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

// Key sources. A source fills a batch of keys at once: k[q] = key j[q] where
// in[q], else 0xffffffff. Every load is issued unmasked (at key 0 in place of
// a masked one) and masked afterwards: a load under a branch is waited for
// inside it, so a batch would arrive one key at a time. ArrayKeys reads an
// array; route_predict_sort's source computes each key from its token.
template <typename KeyT>
struct ArrayKeys {
  const KeyT* __restrict__ p;
  template <int NB>
  __device__ __forceinline__ void batch(const int64_t (&j)[NB], const bool (&in)[NB],
                                        uint32_t (&k)[NB]) const {
    KeyT v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = p[in[q] ? j[q] : 0];
#pragma unroll
    for (int q = 0; q < NB; ++q) k[q] = in[q] ? key_u32<KeyT>(v[q]) : 0xffffffffu;
  }
};

template <typename Src>
__global__ __launch_bounds__(kSortThreads) void csort_hist(Src keys, int64_t n, int B,
                                                           int64_t chunk, int nchunks,
                                                           int* __restrict__ hist, uint32_t* err,
                                                           uint32_t ebit) {
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
    int64_t jq[kBatch];
    bool in[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      jq[q] = j0 + q * kSortThreads;
      in[q] = jq[q] < hi;
    }
    keys.batch(jq, in, k);
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

// Exclusive scan of the B bin totals in tot[] by one wave (each lane a
// contiguous run of bins); *total receives the sum.
__device__ __forceinline__ void scan_bins(int* tot, int B, int* total) {
  const int lane = lane_id();
  const int per = (B + kWave - 1) / kWave;
  const int lo = lane * per;
  const int hi = lo + per < B ? lo + per : B;
  int local = 0;
  for (int b = lo; b < hi; ++b) local += tot[b];
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  int run = incl - local;
  for (int b = lo; b < hi; ++b) {
    const int v = tot[b];
    tot[b] = run;
    run += v;
  }
  if (lane == kWave - 1) *total = incl;
}

// keys [base, base + NB * 64) of a share ending at qhi, one per lane and tile
// (NB tiles)
template <typename Src, int NB>
__device__ __forceinline__ void load_batch(const Src& keys, uint32_t (&kb)[NB], int64_t base,
                                           int64_t qhi) {
  const int lane = lane_id();
  int64_t jq[NB];
  bool in[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    jq[q] = base + q * kWave + lane;
    in[q] = jq[q] < qhi;
  }
  keys.batch(jq, in, kb);
}

// Pass 1 of the ranking: per-bin counts of the keys [qlo, qhi) into this
// wave's LDS row (per 64-key tile, the lowest lane of each key's match adds
// the match size). first[] holds the share's first batch, already loaded.
// Returns whether a key of the share was out of range.
template <typename Src, int NB>
__device__ __forceinline__ bool count_share(const Src& keys, int64_t qlo, int64_t qhi, int B,
                                            int nbits, const uint32_t (&first)[NB],
                                            int* myrow) {
  const int lane = lane_id();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  bool bad = false;
  for (int64_t jb = qlo; jb < qhi; jb += NB * kWave) {
    uint32_t kb[NB];
    if (jb == qlo) {
#pragma unroll
      for (int q = 0; q < NB; ++q) kb[q] = first[q];
    } else {
      load_batch(keys, kb, jb, qhi);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      if (jb + q * kWave >= qhi) break;
      const uint32_t k = kb[q];
      const bool valid = k < static_cast<uint32_t>(B);
      if (!valid && jb + q * kWave + lane < qhi) bad = true;
      const uint64_t m = match_key(k, valid, nbits);
      if (valid && __popcll(m & below) == 0) myrow[k] += __popcll(m);
    }
  }
  return bad;
}

// Pass 2: each key of [qlo, qhi) in order takes its wave's running start for
// its bin plus its rank among equal keys of its tile; the lowest lane of the
// match then advances the start. fwd[j] = position, inv[pos] = j,
// inv_key[pos] = key (nullable); out-of-range keys get position -1.
// With lpos given, each key's position (or -1) also goes to lpos[j - lbase].
template <typename Src, int NB>
__device__ __forceinline__ void place_share(const Src& keys, int64_t qlo, int64_t qhi, int B,
                                            int nbits, const uint32_t (&first)[NB],
                                            int* myrow, int* __restrict__ fwd,
                                            int* __restrict__ inv, uint8_t* __restrict__ inv_key,
                                            int* lpos = nullptr, int64_t lbase = 0) {
  const int lane = lane_id();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t jb = qlo; jb < qhi; jb += NB * kWave) {
    uint32_t kb[NB];
    if (jb == qlo) {
#pragma unroll
      for (int q = 0; q < NB; ++q) kb[q] = first[q];
    } else {
      load_batch(keys, kb, jb, qhi);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
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
        if (lpos) lpos[j - lbase] = pos;
      } else if (j < qhi) {
        fwd[j] = -1;
        if (lpos) lpos[j - lbase] = -1;
      }
      if (valid && rank == 0) myrow[k] = start + __popcll(m);
    }
  }
}

// Ranks the keys of chunk blockIdx.x. fwd[j] = position of key j,
// inv[pos] = j, inv_key[pos] = key (inv_key nullable). THREADS / 64 waves.
//
// Prologue: per bin, the total count and the count in earlier chunks. The
// threads form R = min(THREADS / B, nchunks) groups of B; group r sums chunks
// r, r + R, ... so the loads spread over all threads, and the R partial sums
// meet in LDS.
//
// The chunk is split into NW contiguous shares, one per wave. Pass 1
// (count_share) counts each share per bin into its wave's LDS row. After one
// barrier the rows become per-wave starting positions (the chunk's base for
// the bin plus the counts of the earlier shares). Pass 2 (place_share) walks
// each share again in order. Waves touch only their own LDS row, in program
// order, so pass 2 needs no barriers. More waves make each wave's serial walk
// shorter: the kernel is bound by that walk's latency, not by throughput.
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
  const int c = blockIdx.x;
  for (int i = t; i < NW * B; i += THREADS) wrow[i] = 0;

  // this wave's share of the chunk; its keys are read kBatch tiles (of 64)
  // at a time, and the first batch goes out now, beside the table's loads
  // below (the first batch stays in registers for pass 2)
  const int64_t clo = static_cast<int64_t>(c) * chunk;
  const int64_t chi = clo + chunk < n ? clo + chunk : n;
  const int64_t share = chunk / NW;
  const int64_t qlo = clo + w * share;
  const int64_t qhi = qlo + share < chi ? qlo + share : chi;
  int* myrow = wrow + w * B;
  const ArrayKeys<KeyT> src{keys};
  uint32_t first[kBatch];
  load_batch(src, first, qlo, qhi);

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
  if (w == 0) scan_bins(stot, B, &stotal);
  __syncthreads();
  for (int b = t; b < B; b += THREADS) {
    if (c == 0) offsets[b] = stot[b];
    sbase[b] += stot[b];
  }
  if (c == 0 && t == 0) offsets[B] = stotal;

  count_share(src, qlo, qhi, B, nbits, first, myrow);  // csort_hist flagged bad keys
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
  place_share(src, qlo, qhi, B, nbits, first, myrow, fwd, inv, inv_key);
}

// The whole sort in one workgroup of sixteen waves, for n <= kSortOneMax keys
// and B <= kMaxExperts / 4 bins: the shares of csort_rank span the array, and
// the bin totals come from pass 1's own counts instead of a histogram table.
// One launch instead of two, but one CU's vector units walk every tile, so it
// only pays for small arrays. Measured per sort (graph replay, MI355X), one
// launch against two: 4096 keys of 8 bins 6.5 against 7.1 us, 2048 keys of 4
// bins (with a minimal row move) 7.1 against 8.8; 8192 keys 9.8 against 7.3,
// 16384 keys 17.5 against 7.5 (8 bins) and 28.3 against 9.2 (160 bins).
constexpr int64_t kSortOneMax = 4096;
constexpr int kSortOneThreads = 1024;

template <typename Src>
__global__ __launch_bounds__(kSortOneThreads) void csort_one(
    Src keys, int64_t n, int B, int nbits, int* __restrict__ offsets, int* __restrict__ fwd,
    int* __restrict__ inv, uint8_t* __restrict__ inv_key, uint32_t* err, uint32_t ebit) {
  constexpr int NW = kSortOneThreads / kWave;
  constexpr int kMaxB = kMaxExperts / 4;
  __shared__ int stot[kMaxB];
  __shared__ int wrow[NW * kMaxB];
  __shared__ int stotal;
  const int t = threadIdx.x;
  const int w = wave_id();
  for (int i = t; i < NW * B; i += kSortOneThreads) wrow[i] = 0;
  // shares of whole tiles, one per wave
  const int64_t share = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int64_t qlo = w * share < n ? w * share : n;
  const int64_t qhi = qlo + share < n ? qlo + share : n;
  int* myrow = wrow + w * B;
  uint32_t first[kBatch];
  load_batch(keys, first, qlo, qhi);
  __syncthreads();
  const bool bad = count_share(keys, qlo, qhi, B, nbits, first, myrow);
  if (bad) set_err(err, ebit);
  __syncthreads();
  for (int b = t; b < B; b += kSortOneThreads) {
    int tot = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) tot += wrow[v * B + b];
    stot[b] = tot;
  }
  __syncthreads();
  if (w == 0) scan_bins(stot, B, &stotal);
  __syncthreads();
  // bin starts -> per-wave starting positions
  for (int b = t; b < B; b += kSortOneThreads) {
    offsets[b] = stot[b];
    int run = stot[b];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int cnt = wrow[v * B + b];
      wrow[v * B + b] = run;
      run += cnt;
    }
  }
  if (t == 0) offsets[B] = stotal;
  __syncthreads();
  place_share(keys, qlo, qhi, B, nbits, first, myrow, fwd, inv, inv_key);
}

// Counting every key outside chunk [clo, chi) of [0, n), for kernels that
// rank one chunk each without a histogram table (every workgroup counts the
// whole array for itself, so this pays for small arrays only). Per bin, for
// this wave's share of those keys: the keys before the chunk go to pre[b],
// those after it to post[b], for B <= 8 * NR bins. The keys outside the
// chunk are taken as one range (index j' < clo is key j', else key j' +
// chunk length), split into NW shares of whole tiles, counted a batch of NBO
// keys per lane at a time. Each lane keeps 8-bit counters, eight to a 64-bit
// register (a lane meets at most kCountMaxPerLane keys); the wave's totals
// are summed in 16-bit fields. Out-of-range keys are not counted (their
// owner flags them).
constexpr int kCountMaxPerLane = 255;

// This wave's share of the keys outside the chunk (indices of the joined
// range; NW shares of whole tiles).
template <int NW>
__device__ __forceinline__ void others_share(int64_t n, int64_t clo, int64_t chi, int w,
                                             int64_t* qlo, int64_t* qhi) {
  const int64_t len = n - (chi - clo);
  const int64_t share = ((len + NW - 1) / NW + kWave - 1) / kWave * kWave;
  *qlo = w * share < len ? w * share : len;
  *qhi = *qlo + share < len ? *qlo + share : len;
}

// The first batch of the share [qlo, qhi), NBO keys per lane
// (0xffffffff past the share), so the caller can issue it early. Index
// arithmetic in 32 bits (n < 2^31).
template <typename Src, int NBO>
__device__ __forceinline__ void others_load(const Src& keys, int64_t qlo, int64_t qhi,
                                            int64_t clo, int64_t chi,
                                            uint32_t (&k)[NBO]) {
  const int lane = lane_id();
  const int lo = static_cast<int>(qlo), hi = static_cast<int>(qhi);
  const int c0 = static_cast<int>(clo), gap = static_cast<int>(chi - clo);
  int64_t jq[NBO];
  bool in[NBO];
#pragma unroll
  for (int q = 0; q < NBO; ++q) {
    const int jp = lo + q * kWave + lane;
    in[q] = jp < hi;
    jq[q] = jp < c0 ? jp : jp + gap;
  }
  keys.batch(jq, in, k);
}

// Counts the share, its first batch already in k[] (loaded by others_load).
template <int NR, typename Src, int NBO>
__device__ __forceinline__ void others_count(const Src& keys, int64_t qlo, int64_t qhi,
                                             int64_t clo, int64_t chi, int B,
                                             uint32_t (&k)[NBO], int* pre, int* post) {
  const int lane = lane_id();
  uint64_t cp[NR], cq[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) cp[r] = cq[r] = 0;
  for (int64_t jb = qlo; jb < qhi; jb += NBO * kWave) {
    if (jb != qlo) others_load(keys, jb, qhi, clo, chi, k);
    const int rel = static_cast<int>(jb - clo) + lane;  // < 0: before the chunk
#pragma unroll
    for (int q = 0; q < NBO; ++q) {
      const uint64_t one = k[q] < static_cast<uint32_t>(B) ? 1ull << (8 * (k[q] & 7u)) : 0ull;
      const bool before = rel + q * kWave < 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint64_t add = (k[q] >> 3) == static_cast<uint32_t>(r) ? one : 0ull;
        cp[r] += before ? add : 0ull;
        cq[r] += before ? 0ull : add;
      }
    }
  }
  auto flush = [&](uint64_t c, int r, int* row) {
    // bins 8r + {0, 2, 4, 6} and 8r + {1, 3, 5, 7} as 16-bit fields
    const uint64_t even = c & 0x00ff00ff00ff00ffull;
    const uint64_t odd = (c >> 8) & 0x00ff00ff00ff00ffull;
    const uint32_t s0 = static_cast<uint32_t>(wave_sum_dpp(static_cast<int>(even)));
    const uint32_t s1 = static_cast<uint32_t>(wave_sum_dpp(static_cast<int>(even >> 32)));
    const uint32_t s2 = static_cast<uint32_t>(wave_sum_dpp(static_cast<int>(odd)));
    const uint32_t s3 = static_cast<uint32_t>(wave_sum_dpp(static_cast<int>(odd >> 32)));
    // lane l < 8 takes bin 8r + l: word (l & 1 ? odd : even), half (l & 2)
    const int l = lane & 7;
    const uint32_t word = (l & 1) ? ((l & 4) ? s3 : s2) : ((l & 4) ? s1 : s0);
    const int v = static_cast<int>((l & 2) ? word >> 16 : word & 0xffffu);
    const int b = 8 * r + l;
    if (lane < 8 && b < B) row[b] = v;
  };
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    flush(cp[r], r, pre);
    flush(cq[r], r, post);
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

// Enqueues the sort: one launch up to kSortOneMax keys, else two. ws holds
// the histogram table (unused by the one-launch form). The keys come from
// src; `keys` holds them once src has been read (the rank launch reads them
// there): the same array for a plain sort, the array src writes otherwise.
template <typename KeyT, typename Src>
int csort_launch_src(const Src& src, const KeyT* keys, int64_t n, int B, int* offsets, int* fwd,
                     int* inv, uint8_t* inv_key, void* ws, uint32_t* err, uint32_t ebit,
                     hipStream_t s) {
  if (n == 0) {
    fill_i32<<<ceil_div(B + 1, 256), 256, 0, s>>>(offsets, B + 1, 0);
    return launch_status();
  }
  if (n <= kSortOneMax && B <= kMaxExperts / 4) {
    csort_one<Src><<<1, kSortOneThreads, 0, s>>>(src, n, B, bits_for(B), offsets, fwd, inv,
                                                 inv_key, err, ebit);
    return launch_status();
  }
  const int64_t chunk = csort_chunk(n, B);
  const int nch = static_cast<int>(csort_nchunks(n, B));
  int* hist = static_cast<int*>(ws);
  csort_hist<Src><<<nch, kSortThreads, 0, s>>>(src, n, B, chunk, nch, hist, err, ebit);
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

template <typename KeyT>
int csort_launch(const KeyT* keys, int64_t n, int B, int* offsets, int* fwd, int* inv,
                 uint8_t* inv_key, void* ws, uint32_t* err, uint32_t ebit, hipStream_t s) {
  return csort_launch_src(ArrayKeys<KeyT>{keys}, keys, n, B, offsets, fwd, inv, inv_key, ws, err,
                          ebit, s);
}

}  // namespace
}  // namespace route
