// lar_count and hit_count: the two quality counters of the path.
// Local activation rate: "Speculative MoE" notes, section 7 glossary, and
// the rho of the "Federation of Experts (FoE)" article. Prefetch hit rate:
// "Speculating Experts Accelerates Inference for Mixture-of-Experts",
// technical summary item 4. Integer counts, block-reduced, one 64-bit atomic
// add per block over a capped grid-stride grid.
#include "common.hpp"

namespace route {

constexpr int kCntThreads = 256;
constexpr unsigned kCntMaxBlocks = 128;  // few blocks: few atomics on one address
constexpr int kLarBatch = 8;

// Block-wide sum of one count per thread; thread 0 adds it to *dst.
__device__ __forceinline__ void block_add(unsigned v, unsigned long long* dst) {
  __shared__ unsigned part[kCntThreads / kWave];
  v = wave_sum_u32(v);
  if (lane_id() == 0) part[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
#pragma unroll
    for (int w = 0; w < kCntThreads / kWave; ++w) t += part[w];
    if (t) atomicAdd(dst, static_cast<unsigned long long>(t));
  }
}

__global__ __launch_bounds__(kCntThreads) void lar_kernel(
    const int32_t* __restrict__ idx, int64_t n, int K, int H,
    const uint8_t* __restrict__ row_cluster, const uint8_t* __restrict__ expert_cluster, int E,
    unsigned long long* __restrict__ local) {
  const int kg = K / H;
  const int64_t np = n * K;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCntThreads;
  unsigned hit = 0;
  // kLarBatch pairs a thread at a time, every load of a batch issued before
  // any is used: the grid is capped, so each thread walks many pairs, and one
  // at a time each would wait out two dependent loads
  for (int64_t p0 = static_cast<int64_t>(blockIdx.x) * kCntThreads + threadIdx.x; p0 < np;
       p0 += stride * kLarBatch) {
    int e[kLarBatch];
#pragma unroll
    for (int b = 0; b < kLarBatch; ++b) {
      const int64_t p = p0 + b * stride;
      e[b] = p < np ? idx[p] : -1;
    }
    int ec[kLarBatch], rc[kLarBatch];
#pragma unroll
    for (int b = 0; b < kLarBatch; ++b) {
      const int64_t p = p0 + b * stride;
      const bool ok = e[b] >= 0 && e[b] < E;
      const int64_t i = p / K;
      const int k = static_cast<int>(p - i * K);
      ec[b] = ok ? static_cast<int>(expert_cluster[e[b]]) : -1;
      rc[b] = ok ? static_cast<int>(row_cluster[i * H + k / kg]) : -2;
    }
#pragma unroll
    for (int b = 0; b < kLarBatch; ++b) hit += ec[b] == rc[b] ? 1u : 0u;
  }
  block_add(hit, local);
}

__global__ __launch_bounds__(kCntThreads) void hit_kernel(const int32_t* __restrict__ pred,
                                                          const int32_t* __restrict__ truth,
                                                          int64_t n, int K,
                                                          unsigned long long* __restrict__ hits) {
  unsigned cnt = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCntThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kCntThreads) {
    int t[kMaxK];
    int p[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      t[k] = k < K ? truth[i * K + k] : 0;
      p[k] = k < K ? pred[i * K + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      bool in_truth = false, seen = false;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < K && t[j] == p[k]) in_truth = true;
        if (j < k && p[j] == p[k]) seen = true;
      }
      cnt += (k < K && in_truth && !seen) ? 1u : 0u;
    }
  }
  block_add(cnt, hits);
}

// K a compile-time even number: each row read as K/2 eight-byte vectors,
// all issued before any compare.
template <int KT>
__global__ __launch_bounds__(kCntThreads) void hit_kernel_k(const int32_t* __restrict__ pred,
                                                            const int32_t* __restrict__ truth,
                                                            int64_t n,
                                                            unsigned long long* __restrict__ hits) {
  static_assert(KT % 2 == 0, "pairs of ids per load");
  unsigned cnt = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCntThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kCntThreads) {
    int t[KT], p[KT];
    const int2* tr = reinterpret_cast<const int2*>(truth + i * KT);
    const int2* pr = reinterpret_cast<const int2*>(pred + i * KT);
#pragma unroll
    for (int k = 0; k < KT / 2; ++k) {
      const int2 a = tr[k], b = pr[k];
      t[2 * k] = a.x;
      t[2 * k + 1] = a.y;
      p[2 * k] = b.x;
      p[2 * k + 1] = b.y;
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      bool in_truth = false, seen = false;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        in_truth = in_truth || t[j] == p[k];
        if (j < k) seen = seen || p[j] == p[k];
      }
      cnt += (in_truth && !seen) ? 1u : 0u;
    }
  }
  block_add(cnt, hits);
}

}  // namespace route

using namespace route;

ROUTE_API int lar_count(const int32_t* idx, int64_t n, int32_t K, int32_t H,
                        const uint8_t* row_cluster, const uint8_t* expert_cluster, int32_t E,
                        unsigned long long* local, hipStream_t s) {
  if (n < 0 || K < 1 || H < 1 || K % H != 0 || E < 1) return ROUTE_ERR_SHAPE;
  if (K > kMaxK || E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!idx || !row_cluster || !expert_cluster || !local) return ROUTE_ERR_NULL;
  const unsigned grid = ceil_div(n * K, kCntThreads) < kCntMaxBlocks ? ceil_div(n * K, kCntThreads)
                                                                      : kCntMaxBlocks;
  lar_kernel<<<grid, kCntThreads, 0, s>>>(idx, n, K, H, row_cluster, expert_cluster, E, local);
  return launch_status();
}

ROUTE_API int hit_count(const int32_t* pred, const int32_t* truth, int64_t n, int32_t K,
                        unsigned long long* hits, hipStream_t s) {
  if (n < 0 || K < 1) return ROUTE_ERR_SHAPE;
  if (K > kMaxK) return ROUTE_ERR_UNSUPPORTED;
  if (n == 0) return ROUTE_OK;
  if (!pred || !truth || !hits) return ROUTE_ERR_NULL;
  const unsigned grid = ceil_div(n, kCntThreads) < kCntMaxBlocks ? ceil_div(n, kCntThreads)
                                                                 : kCntMaxBlocks;
  const bool al8 = (reinterpret_cast<uintptr_t>(pred) & 7u) == 0 &&
                   (reinterpret_cast<uintptr_t>(truth) & 7u) == 0;
  if (al8 && K == 8)
    hit_kernel_k<8><<<grid, kCntThreads, 0, s>>>(pred, truth, n, hits);
  else if (al8 && K == 6)
    hit_kernel_k<6><<<grid, kCntThreads, 0, s>>>(pred, truth, n, hits);
  else if (al8 && K == 4)
    hit_kernel_k<4><<<grid, kCntThreads, 0, s>>>(pred, truth, n, hits);
  else if (al8 && K == 2)
    hit_kernel_k<2><<<grid, kCntThreads, 0, s>>>(pred, truth, n, hits);
  else
    hit_kernel<<<grid, kCntThreads, 0, s>>>(pred, truth, n, K, hits);
  return launch_status();
}

ROUTE_API const char* route_status_str(int status) {
  switch (status) {
    case ROUTE_OK: return "ok";
    case ROUTE_ERR_NULL: return "a required pointer is NULL";
    case ROUTE_ERR_SHAPE: return "invalid shape or argument";
    case ROUTE_ERR_ALIGN: return "row data pointer not 16-byte aligned";
    case ROUTE_ERR_UNSUPPORTED: return "size beyond the supported maximum";
    case ROUTE_ERR_WORKSPACE: return "workspace missing or too small";
    case ROUTE_ERR_HIP: return "kernel launch failed";
    case ROUTE_ERR_NOT_MAPPED: return "buffer not device-accessible at its own address";
    default: return "unknown status";
  }
}
