// Token permutation by expert (2kiu.com digest section 3.2: each token's output sums
// the FFNs of its selected experts; section 3.4: tokens travel to the experts' owners
// and none is dropped). On one GPU the dispatch becomes a stable counting sort of the
// (token, slot) pairs by expert, so that each expert's rows are one contiguous segment.
//
// One workgroup of 1024 threads (16 waves). Pass 1 builds the expert histogram in LDS
// and scans it into offsets. Pass 2 walks the tokens in rounds of 1024 (one token per
// thread, in order): each wave ORs its lane bit into a per-(wave, expert) 64-bit mask;
// a token's rank inside its expert is the running base + the popcounts of earlier
// waves' masks + the popcount of its own wave's mask below its lane. Experts are
// distinct within a token, so each mask bit stands for exactly one row.
//
// Shared experts (2kiu.com digest section 3.2 and lpnh.cn guide section 3: one shared
// expert that every token passes through) become extra segments after the routed ones,
// so one grouped-FFN launch serves both: shared expert s owns rows T*k + s*T + t, in
// token order. Rows between the last routed row and T*k (left by topk_idx entries that
// name no routed expert) belong to the first shared segment and carry token -1.
#include "common.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                               int64_t T, int k, int N, int S,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ row_of) {
  __shared__ int hist[kMaxRouted];
  __shared__ int base[kMaxRouted + 1];
  __shared__ unsigned long long mask[kPermWaves][kMaxRouted];
  __shared__ int before[kPermWaves][kMaxRouted];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t pairs = T * k;

  for (int i = tid; i < N; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  for (int64_t p = tid; p < pairs; p += kPermThreads) {
    const int e = idx[p];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < N; ++e) {
      base[e] = run;
      run += hist[e];
    }
    base[N] = run;
  }
  __syncthreads();
  for (int i = tid; i <= N; i += kPermThreads) offsets[i] = base[i];
  for (int s = tid; s < S; s += kPermThreads) offsets[N + 1 + s] = (int32_t)(pairs + (s + 1) * T);
  for (int64_t r = base[N] + tid; r < pairs; r += kPermThreads) row_token[r] = -1;
  for (int64_t r = tid; r < S * T; r += kPermThreads) row_token[pairs + r] = (int32_t)(r % T);

  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t t0 = 0; t0 < T; t0 += kPermThreads) {
    for (int i = tid; i < kPermWaves * N; i += kPermThreads) mask[i / N][i % N] = 0ull;
    __syncthreads();
    const int64_t t = t0 + tid;
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
    for (int e = tid; e < N; e += kPermThreads) {
      int run = 0;
      for (int w = 0; w < kPermWaves; ++w) {
        before[w][e] = run;
        run += __popcll(mask[w][e]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && live) {
        const int e = ej[j];
        int32_t r = -1;
        if (e >= 0) {
          // r < offsets[e] + hist[e] <= T*k: a mask bit never stands for more rows
          // than the histogram counted, even with repeated experts in a token
          r = base[e] + before[wave][e] + __popcll(mask[wave][e] & lt);
          if (r < pairs) row_token[r] = (int32_t)t;
        }
        row_of[t * k + j] = r;
      }
    }
    __syncthreads();
    for (int e = tid; e < N; e += kPermThreads)
      base[e] += before[kPermWaves - 1][e] + __popcll(mask[kPermWaves - 1][e]);
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                                  int32_t* offsets, int32_t* row_token, int32_t* row_of,
                                  void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T * (cfg->top_k + cfg->n_shared) >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (!offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !row_token || !row_of)) return MOE_ERR_NULL;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, as_stream(stream), topk_idx,
                     T, cfg->top_k, cfg->n_routed, cfg->n_shared, offsets, row_token, row_of);
  return launch_status();
}
