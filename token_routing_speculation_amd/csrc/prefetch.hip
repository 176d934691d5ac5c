// Speculative expert prefetch on one GPU: "Speculating Experts Accelerates
// Inference for Mixture-of-Experts", technical summary items 1 (offloaded
// expert weights, on-demand loading after routing), 2 (prefetch the next
// layer's predicted experts during the current layer; speculative execution
// runs them) and 4 (hit rate).
//   prefetch_plan_kernel  : the batch's predicted picks counted per expert in
//       LDS; each named expert's rank (count descending, index ascending)
//       places it in one of C staging slots;
//   prefetch_issue        : host side; the DMA engines copy the listed
//       experts' blocks (hipMemcpyAsync on the caller's copy stream, runs of
//       consecutive experts merged into one transfer). The engines use no
//       compute units and leave concurrent kernels' memory traffic alone;
//   prefetch_copy_kernel  : the same copy as a kernel that reads pinned host
//       memory over PCIe, driven by a device-resident list. It reaches the
//       same link rate, but while it runs concurrent HBM-bound kernels slow
//       down several-fold, so it suits loads made while the GPU waits anyway
//       (on-demand misses after routing), with no host round trip;
//   prefetch_cover_kernel : the true picks whose expert sits in a slot, and
//       the true experts that sit in none (what an on-demand load still
//       copies), listed in index order.
#include "common.hpp"

namespace route {

constexpr int kPfThreads = 1024;  // one workgroup; a thread per expert (E <= 1024)
constexpr int kCopyBlocks = 64;   // the PCIe link saturates at 32-64 workgroups
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kPfThreads) void prefetch_plan_kernel(
    const int32_t* __restrict__ pred, int64_t picks, int E, int C, int32_t* __restrict__ list,
    int32_t* __restrict__ nlist, uint32_t* __restrict__ err) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int wnamed[kPfThreads / kWave];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += kPfThreads) cnt[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int64_t i = t; i < picks; i += kPfThreads) {
    const int p = pred[i];
    if (static_cast<unsigned>(p) < static_cast<unsigned>(E))
      atomicAdd(&cnt[p], 1);
    else
      bad = true;
  }
  if (bad) set_err(err, ROUTE_EBIT_EXPERT_RANGE);
  __syncthreads();
  const int c = t < E ? cnt[t] : 0;
  const int named = wave_sum_dpp(c > 0 ? 1 : 0);
  if (lane_id() == 0) wnamed[wave_id()] = named;
  if (c > 0) {
    // rank among the named experts: those with a larger count, or an equal
    // count and a lower index, come first (cnt[f] read by broadcast)
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int cf = cnt[f];
      rank += (cf > c) | ((cf == c) & (f < t));
    }
    if (rank < C) list[rank] = t;
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kPfThreads / kWave; ++w) total += wnamed[w];
  const int nl = total < C ? total : C;
  for (int i = nl + t; i < C; i += kPfThreads) list[i] = -1;
  if (t == 0) *nlist = nl;
}

__global__ __launch_bounds__(kCopyThreads) void prefetch_copy_kernel(
    const u32x4* __restrict__ bank, int64_t vecs, int E, const int32_t* __restrict__ list, int C,
    u32x4* __restrict__ slots, uint32_t* __restrict__ err) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  for (int i = 0; i < C; ++i) {
    const int e = list[i];
    if (e < 0) continue;  // empty slot
    if (e >= E) {
      if (g == 0) set_err(err, ROUTE_EBIT_EXPERT_RANGE);
      continue;
    }
    const u32x4* src = bank + static_cast<int64_t>(e) * vecs;
    u32x4* dst = slots + static_cast<int64_t>(i) * vecs;
    for (int64_t v = g; v < vecs; v += stride) st16(dst + v, ld16_stream(src + v));
  }
}

__global__ __launch_bounds__(kPfThreads) void prefetch_cover_kernel(
    const int32_t* __restrict__ truth, int64_t picks, int E, const int32_t* __restrict__ list, int C,
    unsigned long long* __restrict__ covered, int32_t* __restrict__ miss,
    int32_t* __restrict__ nmiss, uint32_t* __restrict__ err) {
  __shared__ int inset[kMaxExperts];
  __shared__ int present[kMaxExperts];
  __shared__ unsigned long long wcov[kPfThreads / kWave];
  __shared__ int wmiss[kPfThreads / kWave];
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  for (int e = t; e < E; e += kPfThreads) {
    inset[e] = 0;
    present[e] = 0;
  }
  __syncthreads();
  bool bad = false;
  for (int i = t; i < C; i += kPfThreads) {
    const int e = list[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
      inset[e] = 1;
    else if (e >= E)
      bad = true;
  }
  __syncthreads();
  unsigned long long cov = 0;
  for (int64_t i = t; i < picks; i += kPfThreads) {
    const int p = truth[i];
    if (static_cast<unsigned>(p) < static_cast<unsigned>(E)) {
      present[p] = 1;
      cov += static_cast<unsigned long long>(inset[p]);
    } else {
      bad = true;
    }
  }
  if (bad) set_err(err, ROUTE_EBIT_EXPERT_RANGE);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) cov += __shfl_xor(cov, o, kWave);
  if (lane == 0) wcov[w] = cov;
  __syncthreads();
  // the misses in index order: a ballot prefix within each wave, wave totals after
  const bool flag = t < E && present[t] && !inset[t];
  const unsigned long long ball = __ballot(flag);
  const int below = __popcll(ball & ((1ull << lane) - 1ull));
  if (lane == 0) wmiss[w] = __popcll(ball);
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int q = 0; q < kPfThreads / kWave; ++q) {
    base += q < w ? wmiss[q] : 0;
    total += wmiss[q];
  }
  if (flag) miss[base + below] = t;
  for (int i = total + t; i < E; i += kPfThreads) miss[i] = -1;
  if (t == 0) {
    unsigned long long sum = 0;
#pragma unroll
    for (int q = 0; q < kPfThreads / kWave; ++q) sum += wcov[q];
    atomicAdd(covered, sum);
    *nmiss = total;
  }
}

}  // namespace route

using namespace route;

ROUTE_API int prefetch_plan(const int32_t* pred, int64_t n, int32_t K, int32_t E, int32_t C,
                            int32_t* list, int32_t* nlist, uint32_t* err, hipStream_t s) {
  if (n < 0 || K < 1 || E < 1 || C < 1 || C > E) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if ((n > 0 && !pred) || !list || !nlist) return ROUTE_ERR_NULL;
  prefetch_plan_kernel<<<1, kPfThreads, 0, s>>>(pred, n * K, E, C, list, nlist, err);
  return launch_status();
}

ROUTE_API int prefetch_copy(const void* bank, int32_t E, int64_t expert_bytes, const int32_t* list,
                            int32_t C, void* slots, uint32_t* err, hipStream_t s) {
  if (E < 1 || C < 1 || expert_bytes < 0) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if (expert_bytes % 16 != 0) return ROUTE_ERR_ALIGN;
  if (!bank || !list || !slots) return ROUTE_ERR_NULL;
  if (!aligned16(bank) || !aligned16(slots)) return ROUTE_ERR_ALIGN;
  if (expert_bytes == 0) return ROUTE_OK;
  // the kernel reads the bank directly: it must be device memory or pinned
  // host memory mapped for the device at the same address
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, bank) != hipSuccess) {
    (void)hipGetLastError();
    return ROUTE_ERR_NOT_MAPPED;
  }
  if (at.devicePointer != bank) return ROUTE_ERR_NOT_MAPPED;
  prefetch_copy_kernel<<<kCopyBlocks, kCopyThreads, 0, s>>>(
      static_cast<const u32x4*>(bank), expert_bytes / 16, E, list, C, static_cast<u32x4*>(slots),
      err);
  return launch_status();
}

ROUTE_API int prefetch_coverage(const int32_t* truth, int64_t n, int32_t K, int32_t E,
                                const int32_t* list, int32_t C, unsigned long long* covered,
                                int32_t* miss, int32_t* nmiss, uint32_t* err, hipStream_t s) {
  if (n < 0 || K < 1 || E < 1 || C < 1) return ROUTE_ERR_SHAPE;
  if (E > kMaxExperts) return ROUTE_ERR_UNSUPPORTED;
  if ((n > 0 && !truth) || !list || !covered || !miss || !nmiss) return ROUTE_ERR_NULL;
  prefetch_cover_kernel<<<1, kPfThreads, 0, s>>>(truth, n * K, E, list, C, covered, miss, nmiss,
                                                 err);
  return launch_status();
}

ROUTE_API int prefetch_issue(const void* bank, int32_t E, int64_t expert_bytes,
                             const int32_t* list, int32_t C, void* slots, hipStream_t s) {
  if (E < 1 || C < 1 || expert_bytes < 0) return ROUTE_ERR_SHAPE;
  if (!bank || !list || !slots) return ROUTE_ERR_NULL;
  for (int i = 0; i < C; ++i)  // the host list is checked before anything is enqueued
    if (list[i] < -1 || list[i] >= E) return ROUTE_ERR_SHAPE;
  if (expert_bytes == 0) return ROUTE_OK;
  // asynchronous DMA needs the bank in device memory or in pinned host memory
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, bank) != hipSuccess) {
    (void)hipGetLastError();
    return ROUTE_ERR_NOT_MAPPED;
  }
  if (at.devicePointer == nullptr) return ROUTE_ERR_NOT_MAPPED;
  const char* src = static_cast<const char*>(bank);
  char* dst = static_cast<char*>(slots);
  int i = 0;
  while (i < C) {
    if (list[i] < 0) {
      ++i;
      continue;
    }
    int j = i + 1;  // a run of consecutive experts lands in consecutive slots
    while (j < C && list[j] == list[j - 1] + 1) ++j;
    const size_t bytes = static_cast<size_t>(j - i) * static_cast<size_t>(expert_bytes);
    if (hipMemcpyAsync(dst + static_cast<int64_t>(i) * expert_bytes,
                       src + static_cast<int64_t>(list[i]) * expert_bytes, bytes,
                       hipMemcpyDefault, s) != hipSuccess) {
      (void)hipGetLastError();
      return ROUTE_ERR_HIP;
    }
    i = j;
  }
  return ROUTE_OK;
}

