// Token permutation by expert (2kiu.com digest section 3.2: each token's output sums
// the FFNs of its selected experts; section 3.4: tokens travel to the experts' owners
// and none is dropped). On one GPU the dispatch becomes a stable counting sort of the
// (token, slot) pairs by expert, so that each expert's rows are one contiguous segment.
//
// Three launches over blocks of kPB tokens (one, perm_single_kernel, for a single block):
//   count   - per block, the expert histogram of its pairs (LDS atomics) -> ws[b][e];
//   scan    - one workgroup: per expert, the exclusive prefix over blocks, then the
//             exclusive prefix over experts (offsets, a wave-parallel scan); ws[b][e]
//             becomes the first row
//             of expert e's pairs from block b;
//   scatter - per block, each pair's rank among the block's earlier pairs of the same
//             expert: each wave ORs its lane bit into a per-(wave, expert) 64-bit mask,
//             and a pair's rank is the popcounts of earlier waves' masks plus the
//             popcount of its own wave's mask below its lane. Experts are distinct
//             within a token, so each mask bit stands for exactly one pair.
// Shared experts (2kiu.com digest section 3.2 and lpnh.cn guide section 3: one shared
// expert that every token passes through) become extra segments after the routed ones,
// so one grouped-FFN launch serves both: shared expert s owns rows T*k + s*T + t, in
// token order. Rows between the last routed row and T*k (left by topk_idx entries that
// name no routed expert) belong to the first shared segment and carry token -1.
#include "common.h"

namespace moe {
namespace {

constexpr int kPB = 256;               // tokens per block (4 waves, one token per lane)
constexpr int kPWaves = kPB / kWave;

__global__ __launch_bounds__(kPB) void perm_count_kernel(const int32_t* __restrict__ idx,
                                                         int64_t T, int k, int N,
                                                         int32_t* __restrict__ hist) {
  __shared__ int h[kMaxRouted];
  for (int i = threadIdx.x; i < N; i += kPB) h[i] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPB + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < N) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kPB) hist[(int64_t)blockIdx.x * N + i] = h[i];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(int32_t* __restrict__ hist,
                                                                 int nblk, int N, int S,
                                                                 int64_t T, int64_t pairs,
                                                                 int32_t* __restrict__ offsets) {
  __shared__ int cnt[kMaxRouted];
  __shared__ int base[kMaxRouted + 1];
  const int tid = threadIdx.x;
  // per expert: exclusive prefix of the block counts
  // (8 independent loads per round, so a long column is not one load latency per block)
  for (int e = tid; e < N; e += kScanThreads) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (b0 + u < nblk) ? hist[(int64_t)(b0 + u) * N + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < nblk) hist[(int64_t)(b0 + u) * N + e] = run;
        run += v[u];
      }
    }
    cnt[e] = run;
  }
  __syncthreads();
  // exclusive prefix over experts: per wave by lane shifts, then the wave totals in order
  {
    __shared__ int wtot[kScanThreads / kWave];
    const int lane = tid & (kWave - 1), w = tid / kWave;
    const int v = tid < N ? cnt[tid] : 0;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += u;
    }
    if (lane == kWave - 1) wtot[w] = inc;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += wtot[i];
    if (tid < N) base[tid] = before + inc - v;
    if (tid == N - 1) base[N] = before + inc;
  }
  __syncthreads();
  for (int i = tid; i <= N; i += kScanThreads) offsets[i] = base[i];
  for (int s = tid; s < S; s += kScanThreads) offsets[N + 1 + s] = (int32_t)(pairs + (s + 1) * T);
  for (int64_t i = tid; i < (int64_t)nblk * N; i += kScanThreads)
    hist[i] += base[i % N];
}

__global__ __launch_bounds__(kPB) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                           int64_t T, int k, int N, int S,
                                                           const int32_t* __restrict__ hist,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ row_of) {
  __shared__ unsigned long long mask[kPWaves][kMaxRouted];
  __shared__ int before[kPWaves][kMaxRouted];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t pairs = T * k;
  for (int i = tid; i < kPWaves * N; i += kPB) mask[i / N][i % N] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPB + tid;
  const bool live = t < T;
  int ej[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ej[j] = -1;
    if (j < k && live) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < N) {
        ej[j] = e;
        atomicOr(&mask[wave][e], 1ull << lane);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < N; e += kPB) {
    int run = 0;
    for (int w = 0; w < kPWaves; ++w) {
      before[w][e] = run;
      run += __popcll(mask[w][e]);
    }
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* hb = hist + (int64_t)blockIdx.x * N;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && live) {
      const int e = ej[j];
      int32_t r = -1;
      if (e >= 0) {
        // r < offsets[e] + count[e] <= T*k: a mask bit never stands for more pairs than
        // the histogram counted, even with repeated experts in a token
        r = hb[e] + before[wave][e] + __popcll(mask[wave][e] & lt);
        if (r < pairs) row_token[r] = (int32_t)t;
      }
      row_of[t * k + j] = r;
    }
  }
  // rows past the routed ones: gap rows carry -1, shared segments the token index
  const int64_t stride = (int64_t)gridDim.x * kPB;
  const int64_t v = offsets[N];
  for (int64_t r = v + (int64_t)blockIdx.x * kPB + tid; r < pairs; r += stride) row_token[r] = -1;
  for (int64_t r = (int64_t)blockIdx.x * kPB + tid; r < S * T; r += stride)
    row_token[pairs + r] = (int32_t)(r % T);
}

// A batch of at most kPB tokens (one block: decode): the three steps in one workgroup and
// one launch instead of three, with the same results. The pairs' histogram (LDS atomics,
// as perm_count_kernel), the exclusive prefix over experts (perm_scan_kernel with one
// block, whose per-block prefix is 0), and the stable scatter (perm_scatter_kernel).
__global__ __launch_bounds__(kPB) void perm_single_kernel(const int32_t* __restrict__ idx,
                                                          int64_t T, int k, int N, int S,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ row_of) {
  constexpr int kPer = kMaxRouted / kPB;   // experts per thread in the prefix
  static_assert(kMaxRouted % kPB == 0, "experts per thread");
  __shared__ unsigned long long mask[kPWaves][kMaxRouted];
  __shared__ int before[kPWaves][kMaxRouted];
  __shared__ int cnt[kMaxRouted];
  __shared__ int base[kMaxRouted + 1];
  __shared__ int wtot[kPWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t pairs = T * k;
  for (int i = tid; i < kPWaves * N; i += kPB) mask[i / N][i % N] = 0ull;
  for (int i = tid; i < N; i += kPB) cnt[i] = 0;
  __syncthreads();
  const bool live = tid < T;
  int ej[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ej[j] = -1;
    if (j < k && live) {
      const int e = idx[(int64_t)tid * k + j];
      if (e >= 0 && e < N) {
        ej[j] = e;
        atomicAdd(&cnt[e], 1);
        atomicOr(&mask[wave][e], 1ull << lane);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < N; e += kPB) {
    int run = 0;
    for (int w = 0; w < kPWaves; ++w) {
      before[w][e] = run;
      run += __popcll(mask[w][e]);
    }
  }
  {
    // exclusive prefix of the counts: thread t owns experts kPer*t .. kPer*t + kPer - 1
    int c[kPer], sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = kPer * tid + u;
      c[u] = e < N ? cnt[e] : 0;
      sum += c[u];
    }
    int inc = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += v;
    }
    if (lane == kWave - 1) wtot[wave] = inc;
    __syncthreads();
    int bef = 0;
    for (int i = 0; i < wave; ++i) bef += wtot[i];
    int ex = bef + inc - sum;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = kPer * tid + u;
      if (e < N) base[e] = ex;
      ex += c[u];
    }
    if (tid == kPB - 1) base[N] = bef + inc;   // the total (experts past N add 0)
  }
  __syncthreads();
  for (int i = tid; i <= N; i += kPB) offsets[i] = base[i];
  for (int s = tid; s < S; s += kPB) offsets[N + 1 + s] = (int32_t)(pairs + (s + 1) * T);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && live) {
      const int e = ej[j];
      int32_t r = -1;
      if (e >= 0) {
        r = base[e] + before[wave][e] + __popcll(mask[wave][e] & lt);
        if (r < pairs) row_token[r] = tid;
      }
      row_of[(int64_t)tid * k + j] = r;
    }
  }
  // rows past the routed ones: gap rows carry -1, shared segments the token index
  for (int64_t r = base[N] + tid; r < pairs; r += kPB) row_token[r] = -1;
  for (int64_t r = tid; r < S * T; r += kPB) row_token[pairs + r] = (int32_t)(r % T);
}

inline int64_t perm_blocks(int64_t T) { return (T + kPB - 1) / kPB; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_config(cfg) != MOE_OK || T <= 0) return 0;
  return (size_t)perm_blocks(T) * cfg->n_routed * sizeof(int32_t);
}

extern "C" moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                                  int32_t* offsets, int32_t* row_token, int32_t* row_of,
                                  void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T * (cfg->top_k + cfg->n_shared) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (!offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !row_token || !row_of)) return MOE_ERR_NULL;
  const int64_t nblk = perm_blocks(T);
  if (T > 0 && (!ws || ws_bytes < (size_t)nblk * cfg->n_routed * sizeof(int32_t)))
    return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int N = cfg->n_routed, k = cfg->top_k, S = cfg->n_shared;
  int32_t* hist = static_cast<int32_t*>(ws);
  if (T > 0 && T <= kPB) {
    hipLaunchKernelGGL(perm_single_kernel, dim3(1), dim3(kPB), 0, s, topk_idx, T, k, N, S, offsets,
                       row_token, row_of);
    return launch_status();
  }
  if (T > 0)
    hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nblk), dim3(kPB), 0, s, topk_idx, T, k, N,
                       hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, hist, (int)nblk, N, S, T,
                     T * k, offsets);
  if (T > 0)
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)nblk), dim3(kPB), 0, s, topk_idx, T, k,
                       N, S, hist, offsets, row_token, row_of);
  return launch_status();
}
