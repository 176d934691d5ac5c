// Speculative expert grouping (s-EG): "Speculative MoE" notes, section 3.2
// (experts that the same tokens activate together share a cluster; placed
// offline, the gate's columns permuted to match) and section 4.2 (balanced
// token-expert co-clustering: a theta-weighted sum of the token-load
// imbalance and of the activations that cross clusters, equal experts per
// cluster, solved by a two-stage cross-entropy method).
//
// The solve is a sequence of launches with no host round trip, so one
// iteration (sample -> score -> update) can be replayed as a HIP graph:
//   eg_profile : token-id x expert activation counts of a routed batch
//                (integer atomics: exact in any order);
//   eg_sample  : B candidate placements drawn expert by expert from P[e][g]
//                among the clusters with room left (counter-based SplitMix64);
//   eg_score   : S_b = counts . onehot(place_b) for all b at once, on the
//                bf16 matrix cores: the counts split into their high and low
//                bytes (both exact in bf16) along K, the one-hot columns
//                carrying 256 and 1, so every product and every partial sum
//                is an integer below 2^24 and the binary32 result is exact;
//                then each token's best cluster (lowest on ties) gives
//                local[b] and the token loads load[b][g] (two-stage integer
//                reduction, no atomics);
//   eg_update  : the objective J, the elite set (ties to the lower index),
//                P <- alpha * elite frequency + (1 - alpha) * P, and the best
//                placement seen.
// Float64 steps follow the written operation order (contraction is off in
// this file), so they are reproducible and match a plain definition bit for
// bit.
#include "common.hpp"
#include "gemm.hpp"

#pragma clang fp contract(off)

namespace route {

constexpr int kEgThreads = 256;
constexpr int kEgMaxG = 32;
constexpr int kEgMaxB = 1024;
constexpr int kEgRowsPerBlock = 8;    // tokens per block in the score reduction
constexpr int kEgUpdateLdsBytes = 32768;  // elite placements staged in LDS up to this
constexpr int kEgSampleThreads = 32;  // candidates per block in the sampler
constexpr int kEgSampleLdsDoubles = 4096;  // P staged in LDS up to E * G of this

// ------------------------------------------------------------------- profile
__global__ __launch_bounds__(kEgThreads) void eg_profile_kernel(
    const int* __restrict__ tok, const int* __restrict__ idx, int64_t n, int K,
    const int* __restrict__ row_of_id, int vocab, int U, int E, int* __restrict__ counts,
    int* __restrict__ freq, uint32_t* err) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kEgThreads + threadIdx.x;
  if (t >= n * K) return;
  const int64_t i = t / K;
  const int k = static_cast<int>(t - i * K);
  const int v = tok[i];
  if (v < 0 || v >= vocab) {
    set_err(err, ROUTE_EBIT_TOKEN_RANGE);
    return;
  }
  const int u = row_of_id[v];
  if (u < 0 || u >= U) {
    set_err(err, ROUTE_EBIT_INDEX_RANGE);
    return;
  }
  if (k == 0) atomicAdd(&freq[u], 1);
  const int e = idx[t];
  if (e < 0 || e >= E) {
    set_err(err, ROUTE_EBIT_EXPERT_RANGE);
    return;
  }
  atomicAdd(&counts[static_cast<int64_t>(u) * E + e], 1);
}

// ------------------------------------------------------------------ sampler
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long seed,
                                                         unsigned long long n) {
  unsigned long long z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One thread per candidate b: experts in index order; expert e goes to
// cluster g with probability P[e][g] / W among the clusters with room left
// (W their total): the first g whose running sum exceeds u * W. GM >= G is a
// compile-time bound so the capacities live in registers; sums run over
// g < G in index order. The table is staged in LDS when it fits (each step of
// a walk reads one row of it).
template <bool LDS_P, int GM, bool EXACT>
__global__ __launch_bounds__(kEgSampleThreads) void eg_sample_kernel(
    const double* __restrict__ P, int E, int G_, int B, unsigned long long seed, int iter,
    uint8_t* __restrict__ place) {
  const int G = EXACT ? GM : G_;  // EXACT: G == GM, every bound below folds away
  __shared__ double sP[LDS_P ? kEgSampleLdsDoubles : 1];
  const int t = threadIdx.x;
  if (LDS_P) {
    for (int i = t; i < E * G; i += kEgSampleThreads) sP[i] = P[i];
    __syncthreads();
  }
  const double* Pt = LDS_P ? sP : P;
  const int b = blockIdx.x * kEgSampleThreads + t;
  if (b >= B) return;  // no barrier below: every thread works alone
  int cap[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) cap[g] = g < G ? E / G : 0;
  uint8_t* out = place + static_cast<int64_t>(b) * E;
  // draw n for expert e of this candidate; the walk does not feed the
  // generator, so each step computes the next draw alongside its own sums
  const unsigned long long n0 =
      (static_cast<unsigned long long>(iter) * B + b) * static_cast<unsigned long long>(E) + 1;
  auto draw = [&](int e) {
    return static_cast<double>(splitmix64(seed, n0 + e) >> 11) * 0x1.0p-53;
  };
  double u = draw(0);
  for (int e = 0; e < E; ++e) {
    const double u_next = draw(e + 1 < E ? e + 1 : e);
    const double* pe = Pt + static_cast<int64_t>(e) * G;
    double w[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) w[g] = g < G ? pe[g] : 0.0;
#pragma unroll
    for (int g = 0; g < GM; ++g) w[g] = cap[g] > 0 ? w[g] : 0.0;
    double W = 0.0;
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < G) W = W + w[g];
    const double target = u * W;
    int pick = -1, last_pos = -1, first_open = -1;
    double c = 0.0;
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g < G) {
        c = c + w[g];
        if (pick < 0 && w[g] > 0.0 && c > target) pick = g;
        if (w[g] > 0.0) last_pos = g;
        if (cap[g] > 0 && first_open < 0) first_open = g;
      }
    }
    if (pick < 0) pick = W > 0.0 ? last_pos : first_open;
    out[e] = static_cast<uint8_t>(pick);
#pragma unroll
    for (int g = 0; g < GM; ++g) cap[g] -= g == pick ? 1 : 0;
    u = u_next;
  }
}

template <bool LDS_P, int GM>
static void launch_sample_g(int E, int G, int B, unsigned long long seed, int iter,
                            const double* P, uint8_t* place, hipStream_t s) {
  const unsigned grid = ceil_div(B, kEgSampleThreads);
  if (G == GM)
    eg_sample_kernel<LDS_P, GM, true><<<grid, kEgSampleThreads, 0, s>>>(P, E, G, B, seed, iter,
                                                                       place);
  else
    eg_sample_kernel<LDS_P, GM, false><<<grid, kEgSampleThreads, 0, s>>>(P, E, G, B, seed, iter,
                                                                        place);
}

template <bool LDS_P>
static void launch_sample(int E, int G, int B, unsigned long long seed, int iter, const double* P,
                          uint8_t* place, hipStream_t s) {
  if (G <= 2)
    launch_sample_g<LDS_P, 2>(E, G, B, seed, iter, P, place, s);
  else if (G <= 4)
    launch_sample_g<LDS_P, 4>(E, G, B, seed, iter, P, place, s);
  else if (G <= 8)
    launch_sample_g<LDS_P, 8>(E, G, B, seed, iter, P, place, s);
  else if (G <= 16)
    launch_sample_g<LDS_P, 16>(E, G, B, seed, iter, P, place, s);
  else
    launch_sample_g<LDS_P, 32>(E, G, B, seed, iter, P, place, s);
}

// -------------------------------------------------------------------- score
__device__ __forceinline__ uint16_t bf16_small_int(int c) {  // 0 <= c < 256: exact
  return static_cast<uint16_t>(__float_as_uint(static_cast<float>(c)) >> 16);
}

// A2[u][e] = high byte of counts[u][e], A2[u][E + e] = low byte (as bf16);
// one wave per token row. A count outside [0, 65535], or a row summing to
// 2^24 or more (the bound for exact binary32 sums), sets VALUE_RANGE.
__global__ __launch_bounds__(kEgThreads) void eg_split_kernel(const int* __restrict__ counts,
                                                              int U, int E,
                                                              uint16_t* __restrict__ a2,
                                                              uint32_t* err) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * (kEgThreads / kWave) + wave_id();
  if (u >= U) return;
  const int lane = lane_id();
  const int* row = counts + u * E;
  uint16_t* out = a2 + u * 2 * static_cast<int64_t>(E);
  unsigned sum = 0;
  bool bad = false;
  for (int e = lane; e < E; e += kWave) {
    int c = row[e];
    if (c < 0 || c > 65535) {
      bad = true;
      c = c < 0 ? 0 : 65535;
    }
    sum += static_cast<unsigned>(c);
    out[e] = bf16_small_int(c >> 8);
    out[E + e] = bf16_small_int(c & 255);
  }
  sum = wave_sum_u32(sum);  // at most 1024 * 65535 < 2^32
  if (bad || sum >= (1u << 24)) set_err(err, ROUTE_EBIT_VALUE_RANGE);
}

// B2[b G + g][e] = 256 and B2[b G + g][E + e] = 1 where place[b][e] == g, 0
// elsewhere. A placement entry >= G sets VALUE_RANGE (its expert then counts
// for no cluster).
__global__ __launch_bounds__(kEgThreads) void eg_onehot_kernel(const uint8_t* __restrict__ place,
                                                               int B, int E, int G,
                                                               uint16_t* __restrict__ b2,
                                                               uint32_t* err) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kEgThreads + threadIdx.x;
  const int64_t total = static_cast<int64_t>(B) * G * 2 * E;
  if (t >= total) return;
  const int64_t r = t / (2 * E);
  const int j = static_cast<int>(t - r * 2 * E);
  const int b = static_cast<int>(r / G);
  const int g = static_cast<int>(r - static_cast<int64_t>(b) * G);
  const int e = j < E ? j : j - E;
  const int x = place[static_cast<int64_t>(b) * E + e];
  if (x >= G && g == 0 && j < E) set_err(err, ROUTE_EBIT_VALUE_RANGE);
  const uint16_t one = j < E ? 0x4380u : 0x3F80u;  // 256.0 and 1.0
  b2[t] = x == g ? one : static_cast<uint16_t>(0);
}

// Stage 1 of the reduction: thread = candidate b, block = kEgRowsPerBlock
// tokens (all their sums loaded before any is used); each token's first
// maximum over its G cluster sums. Writes this block's partial
// [local, load[0..G-1]] per candidate.
template <int GM>
__global__ __launch_bounds__(kEgThreads) void eg_reduce_kernel(const float* __restrict__ S,
                                                               const int* __restrict__ freq,
                                                               int U, int G, int B,
                                                               long long* __restrict__ part) {
  const int b = blockIdx.y * kEgThreads + threadIdx.x;
  if (b >= B) return;
  const int u0 = blockIdx.x * kEgRowsPerBlock;
  const int64_t ld = static_cast<int64_t>(B) * G;
  float v[kEgRowsPerBlock][GM];
  long long f[kEgRowsPerBlock];
#pragma unroll
  for (int q = 0; q < kEgRowsPerBlock; ++q) {
    const int u = u0 + q < U ? u0 + q : U - 1;  // past the end: reload the last row, unused
    const float* s = S + u * ld + static_cast<int64_t>(b) * G;
#pragma unroll
    for (int g = 0; g < GM; ++g) v[q][g] = g < G ? s[g] : 0.f;
    f[q] = freq[u];
  }
  long long loc = 0;
  long long lo[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) lo[g] = 0;
#pragma unroll
  for (int q = 0; q < kEgRowsPerBlock; ++q) {
    if (u0 + q >= U) break;
    float best = v[q][0];
    int bg = 0;
#pragma unroll
    for (int g = 1; g < GM; ++g) {
      if (g < G && v[q][g] > best) {  // strict: the lowest g on equal sums
        best = v[q][g];
        bg = g;
      }
    }
    loc += static_cast<long long>(best);
#pragma unroll
    for (int g = 0; g < GM; ++g) lo[g] += g == bg ? f[q] : 0;
  }
  long long* out = part + (static_cast<int64_t>(blockIdx.x) * B + b) * (G + 1);
  out[0] = loc;
#pragma unroll
  for (int g = 0; g < GM; ++g)
    if (g < G) out[1 + g] = lo[g];
}

// Stage 2: one wave per output sums the blocks' partials (integer sums: the
// order does not change the result).
__global__ __launch_bounds__(kEgThreads) void eg_finish_kernel(const long long* __restrict__ part,
                                                               int nblk, int G, int B,
                                                               long long* __restrict__ local,
                                                               long long* __restrict__ load) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kEgThreads / kWave) + wave_id();
  if (t >= static_cast<int64_t>(B) * (G + 1)) return;
  const int b = static_cast<int>(t / (G + 1));
  const int q = static_cast<int>(t - static_cast<int64_t>(b) * (G + 1));
  long long acc = 0;
  for (int k = lane_id(); k < nblk; k += kWave)
    acc += part[(static_cast<int64_t>(k) * B + b) * (G + 1) + q];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (lane_id() == 0) {
    if (q == 0)
      local[b] = acc;
    else
      load[static_cast<int64_t>(b) * G + q - 1] = acc;
  }
}

// ------------------------------------------------------------------- update
__global__ __launch_bounds__(kEgMaxB) void eg_update_kernel(
    const long long* __restrict__ local, const long long* __restrict__ load,
    const uint8_t* __restrict__ place, int B, int E, int G, long long T, long long F,
    double theta, int n_elite, double alpha, double* __restrict__ P, double* __restrict__ best_J,
    uint8_t* __restrict__ best_place, double* __restrict__ Jout) {
  __shared__ double sJ[kEgMaxB];
  __shared__ unsigned char elite[kEgMaxB];
  __shared__ int erank[kEgMaxB];  // elite rank -> candidate
  __shared__ uint8_t eplace[kEgUpdateLdsBytes];
  __shared__ int sbmin;
  __shared__ int improved;
  const int t = threadIdx.x;
  for (int b = t; b < B; b += kEgMaxB) {
    long long m = load[static_cast<int64_t>(b) * G];
    for (int g = 1; g < G; ++g) {
      const long long v = load[static_cast<int64_t>(b) * G + g];
      m = v > m ? v : m;
    }
    const double r = 1.0 - static_cast<double>(local[b]) / static_cast<double>(T);
    const double bal = static_cast<double>(G) * static_cast<double>(m) / static_cast<double>(F) - 1.0;
    const double J = (1.0 - theta) * r + theta * bal;
    sJ[b] = J;
    if (Jout) Jout[b] = J;
  }
  __syncthreads();
  for (int b = t; b < B; b += kEgMaxB) {
    const double Jb = sJ[b];
    int rank = 0;
    for (int c = 0; c < B; ++c) rank += (sJ[c] < Jb || (c < b && sJ[c] == Jb)) ? 1 : 0;
    elite[b] = rank < n_elite ? 1 : 0;
    if (rank < n_elite) erank[rank] = b;
    if (rank == 0) sbmin = b;
  }
  __syncthreads();
  // the elite placements, in rank order, staged in LDS when they fit
  const bool staged = static_cast<int64_t>(n_elite) * E <= kEgUpdateLdsBytes;
  if (staged) {
    for (int i = t; i < n_elite * E; i += kEgMaxB) {
      const int r = i / E;
      eplace[i] = place[static_cast<int64_t>(erank[r]) * E + (i - r * E)];
    }
  }
  __syncthreads();
  for (int i = t; i < E * G; i += kEgMaxB) {
    const int e = i / G;
    const int g = i - e * G;
    int cnt = 0;
    if (staged) {
      for (int r = 0; r < n_elite; ++r) cnt += eplace[r * E + e] == g ? 1 : 0;
    } else {
      for (int b = 0; b < B; ++b)
        cnt += (elite[b] && place[static_cast<int64_t>(b) * E + e] == g) ? 1 : 0;
    }
    const double share = static_cast<double>(cnt) / static_cast<double>(n_elite);
    P[i] = alpha * share + (1.0 - alpha) * P[i];
  }
  if (t == 0) {
    improved = sJ[sbmin] < best_J[0] ? 1 : 0;
    if (improved) best_J[0] = sJ[sbmin];
  }
  __syncthreads();
  if (improved)
    for (int e = t; e < E; e += kEgMaxB) best_place[e] = place[static_cast<int64_t>(sbmin) * E + e];
}

__global__ void fill_i64(long long* __restrict__ p, int64_t n, long long v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void fill_f64(double* __restrict__ p, int64_t n, double v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------- sizes
inline bool eg_shape_ok(int U, int E, int G) {
  return U >= 0 && E >= 4 && E % 4 == 0 && G >= 1 && E % G == 0;
}

struct EgWs {
  size_t a2, b2, s, part, total;
};

inline EgWs eg_ws_layout(int U, int E, int G, int B) {
  EgWs w;
  const size_t nblk = (static_cast<size_t>(U) + kEgRowsPerBlock - 1) / kEgRowsPerBlock;
  w.a2 = 0;
  w.b2 = align_up(w.a2 + static_cast<size_t>(U) * 2 * E * sizeof(uint16_t), 256);
  w.s = align_up(w.b2 + static_cast<size_t>(B) * G * 2 * E * sizeof(uint16_t), 256);
  w.part = align_up(w.s + static_cast<size_t>(U) * B * G * sizeof(float), 256);
  w.total = align_up(w.part + nblk * B * (G + 1) * sizeof(long long), 256);
  return w;
}

}  // namespace route

using namespace route;

ROUTE_API int eg_profile(const int32_t* tok, const int32_t* idx, int64_t n, int32_t K,
                         const int32_t* row_of_id, int32_t vocab, int32_t U, int32_t E,
                         int32_t* counts, int32_t* freq, uint32_t* err, hipStream_t s) {
  if (n < 0 || K < 1 || vocab < 1 || U < 0 || E < 1) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!tok || !idx || !row_of_id || !counts || !freq) return ROUTE_ERR_NULL;
  eg_profile_kernel<<<ceil_div(n * K, kEgThreads), kEgThreads, 0, s>>>(
      tok, idx, n, K, row_of_id, vocab, U, E, counts, freq, err);
  return launch_status();
}

ROUTE_API int eg_sample(const double* P, int32_t E, int32_t G, int32_t B, uint64_t seed,
                        int32_t iter, uint8_t* place, hipStream_t s) {
  if (!eg_shape_ok(0, E, G) || B < 1 || iter < 0) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || G > kEgMaxG || B > kEgMaxB) return ROUTE_ERR_UNSUPPORTED;
  if (!P || !place) return ROUTE_ERR_NULL;
  if (E * G <= kEgSampleLdsDoubles)
    launch_sample<true>(E, G, B, seed, iter, P, place, s);
  else
    launch_sample<false>(E, G, B, seed, iter, P, place, s);
  return launch_status();
}

ROUTE_API size_t eg_score_workspace_size(int32_t U, int32_t E, int32_t G, int32_t B) {
  if (!eg_shape_ok(U, E, G) || B < 1) return 0;
  return eg_ws_layout(U, E, G, B).total;
}

ROUTE_API int eg_score(const int32_t* counts, const int32_t* freq, int32_t U, int32_t E,
                       int32_t G, const uint8_t* place, int32_t B, long long* local,
                       long long* load, void* ws, size_t ws_bytes, uint32_t* err,
                       hipStream_t s) {
  if (!eg_shape_ok(U, E, G) || B < 1) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || G > kEgMaxG || B > kEgMaxB) return ROUTE_ERR_UNSUPPORTED;
  if (!place || !local || !load) return ROUTE_ERR_NULL;
  if (U == 0) {  // no tokens: nothing local, no load
    fill_i64<<<ceil_div(B, 256), 256, 0, s>>>(local, B, 0);
    fill_i64<<<ceil_div(static_cast<int64_t>(B) * G, 256), 256, 0, s>>>(
        load, static_cast<int64_t>(B) * G, 0);
    return launch_status();
  }
  if (!counts || !freq) return ROUTE_ERR_NULL;
  const EgWs w = eg_ws_layout(U, E, G, B);
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return ROUTE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  uint16_t* a2 = reinterpret_cast<uint16_t*>(base + w.a2);
  uint16_t* b2 = reinterpret_cast<uint16_t*>(base + w.b2);
  float* S = reinterpret_cast<float*>(base + w.s);
  long long* part = reinterpret_cast<long long*>(base + w.part);
  eg_split_kernel<<<ceil_div(U, kEgThreads / kWave), kEgThreads, 0, s>>>(counts, U, E, a2, err);
  eg_onehot_kernel<<<ceil_div(static_cast<int64_t>(B) * G * 2 * E, kEgThreads), kEgThreads, 0,
                     s>>>(place, B, E, G, b2, err);
  int st = launch_status();
  if (st != ROUTE_OK) return st;
  st = gemm_f32(a2, U, 2 * E, b2, B * G, S, s);
  if (st != ROUTE_OK) return st;
  const int nblk = static_cast<int>(ceil_div(U, kEgRowsPerBlock));
  dim3 grid(nblk, ceil_div(B, kEgThreads));
  if (G <= 2)
    eg_reduce_kernel<2><<<grid, kEgThreads, 0, s>>>(S, freq, U, G, B, part);
  else if (G <= 4)
    eg_reduce_kernel<4><<<grid, kEgThreads, 0, s>>>(S, freq, U, G, B, part);
  else if (G <= 8)
    eg_reduce_kernel<8><<<grid, kEgThreads, 0, s>>>(S, freq, U, G, B, part);
  else if (G <= 16)
    eg_reduce_kernel<16><<<grid, kEgThreads, 0, s>>>(S, freq, U, G, B, part);
  else
    eg_reduce_kernel<32><<<grid, kEgThreads, 0, s>>>(S, freq, U, G, B, part);
  eg_finish_kernel<<<ceil_div(static_cast<int64_t>(B) * (G + 1), kEgThreads / kWave), kEgThreads,
                     0, s>>>(part, nblk, G, B, local, load);
  return launch_status();
}

ROUTE_API int eg_update(const long long* local, const long long* load, const uint8_t* place,
                        int32_t B, int32_t E, int32_t G, long long total, long long tokens,
                        double theta, int32_t n_elite, double alpha, double* P, double* best_J,
                        uint8_t* best_place, double* J, hipStream_t s) {
  if (!eg_shape_ok(0, E, G) || B < 1 || n_elite < 1 || n_elite > B || total < 1 || tokens < 1)
    return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || G > kEgMaxG || B > kEgMaxB) return ROUTE_ERR_UNSUPPORTED;
  if (!local || !load || !place || !P || !best_J || !best_place) return ROUTE_ERR_NULL;
  eg_update_kernel<<<1, kEgMaxB, 0, s>>>(local, load, place, B, E, G, total, tokens, theta,
                                         n_elite, alpha, P, best_J, best_place, J);
  return launch_status();
}

ROUTE_API int eg_init(double* P, int32_t E, int32_t G, double* best_J, hipStream_t s) {
  if (!eg_shape_ok(0, E, G)) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts || G > kEgMaxG) return ROUTE_ERR_UNSUPPORTED;
  if (!P || !best_J) return ROUTE_ERR_NULL;
  fill_f64<<<ceil_div(static_cast<int64_t>(E) * G, 256), 256, 0, s>>>(
      P, static_cast<int64_t>(E) * G, 1.0 / static_cast<double>(G));
  fill_f64<<<1, 1, 0, s>>>(best_J, 1, __builtin_inf());
  return launch_status();
}
