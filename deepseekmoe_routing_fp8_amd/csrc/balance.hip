// Per-sequence balance statistics of one routing step (2kiu.com digest section 3.3: a
// complementary sequence-level balance loss, alpha times the sum over experts of the
// expert's share of the sequence's assignments times its mean affinity in the sequence;
// section 5.5: the per-sequence allocation entropy is what to watch before relying on
// that loss). Sequences are runs of L consecutive tokens.
//
//   f_i = (pairs of the sequence routed to expert i) / (k L)
//   P_i = (1/L) * sum over the sequence's tokens of the sigmoid affinity s_{t,i}
//   loss = alpha * sum_i f_i P_i,   entropy = -sum_{f_i > 0} f_i ln f_i
//
// Two launches, both deterministic (fixed summation order, integer histograms):
//   partial  - one workgroup per (sequence, chunk of kSC tokens): per expert, the FP64
//              sum of the chunk's affinities (a thread owns expert columns, so each token
//              row is read coalesced) and the chunk's assignment histogram (LDS integer
//              atomics) -> workspace;
//   finalise - one workgroup per sequence: per expert, the chunk sums (four contiguous
//              runs of chunks in parallel, then the four run totals in order), then
//              f_i P_i and -f_i ln f_i reduced over experts in a fixed order (lane
//              butterflies, then waves in order) in FP64, rounded once to FP32.
#include "common.h"

namespace moe {
namespace {

constexpr int kSC = 32;          // tokens per partial workgroup
constexpr int kBT = 256;         // threads per workgroup
constexpr int kEPT = kMaxRouted / kBT;   // expert columns per thread
constexpr int kRB = 16;          // score rows loaded per round in the partial kernel
constexpr int kFB = 16;          // chunk partials loaded per round in the finalise kernel
constexpr int kFT = 1024;        // finalise threads: kFG groups of kBT
constexpr int kFG = kFT / kBT;

__global__ __launch_bounds__(kBT) void seqbal_partial_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ idx,
                                                             int64_t L, int64_t nch, int N, int k,
                                                             double* __restrict__ psum,
                                                             int32_t* __restrict__ pcnt) {
  __shared__ int h[kMaxRouted];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;                 // = q * nch + c
  const int64_t q = blk / nch, c = blk % nch;
  const int64_t t0 = q * L + c * kSC;
  const int nt = (int)(L - c * kSC < kSC ? L - c * kSC : kSC);
  for (int e = tid; e < N; e += kBT) h[e] = 0;
  __syncthreads();
  for (int p = tid; p < nt * k; p += kBT) {
    const int e = idx[t0 * k + p];
    if (e >= 0 && e < N) atomicAdd(&h[e], 1);
  }
  double acc[kEPT];
#pragma unroll
  for (int j = 0; j < kEPT; ++j) acc[j] = 0.0;
  const float* row = scores + t0 * N;
  // kRB rows in flight per round, summed in token order. Row indices past the chunk are
  // clamped to its last row and their values dropped, so every load is unconditional and
  // the round's loads issue back to back.
  for (int r0 = 0; r0 < nt; r0 += kRB) {
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
      const int e = tid + j * kBT;
      if (e < N) {
        float v[kRB];
#pragma unroll
        for (int u = 0; u < kRB; ++u) v[u] = row[(int64_t)min(r0 + u, nt - 1) * N + e];
#pragma unroll
        for (int u = 0; u < kRB; ++u) acc[j] += (r0 + u < nt) ? (double)v[u] : 0.0;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    const int e = tid + j * kBT;
    if (e < N) {
      psum[blk * N + e] = acc[j];
      pcnt[blk * N + e] = h[e];
    }
  }
}

// Butterfly sum over the 64 lanes of a wave (a fixed pattern: deterministic).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// One workgroup per sequence: kFG groups of kBT threads each sum a contiguous quarter of
// the chunk partials (kFB loads in flight per round), the group totals are added in group
// order, then the per-expert terms are reduced over the block.
__global__ __launch_bounds__(kFT) void seqbal_final_kernel(const double* __restrict__ psum,
                                                           const int32_t* __restrict__ pcnt,
                                                           int64_t L, int64_t nch, int N, int k,
                                                           double alpha, float* __restrict__ loss,
                                                           float* __restrict__ entropy) {
  __shared__ double gsum[kFG][kMaxRouted];
  __shared__ int gcnt[kFG][kMaxRouted];
  __shared__ double red[2][kFT / kWave];
  const int tid = threadIdx.x, g = tid / kBT, el = tid % kBT;
  const int64_t q = blockIdx.x;
  const int64_t per = (nch + kFG - 1) / kFG;
  const int64_t cb = g * per, ce = (cb + per < nch) ? cb + per : nch;
  for (int j = 0; j < kEPT; ++j) {
    const int e = el + j * kBT;
    if (e >= N) break;
    double s = 0.0;
    int cnt = 0;
    for (int64_t c0 = cb; c0 < ce; c0 += kFB) {
      double ps[kFB];
      int32_t pc[kFB];
#pragma unroll
      for (int u = 0; u < kFB; ++u) {   // clamped like the partial kernel's rows
        const int64_t o = (q * nch + (c0 + u < ce ? c0 + u : ce - 1)) * N + e;
        ps[u] = psum[o];
        pc[u] = pcnt[o];
      }
#pragma unroll
      for (int u = 0; u < kFB; ++u) {
        const bool in = c0 + u < ce;
        s += in ? ps[u] : 0.0;
        cnt += in ? pc[u] : 0;
      }
    }
    gsum[g][e] = s;
    gcnt[g][e] = cnt;
  }
  __syncthreads();
  const double kl = (double)k * (double)L;
  double lsum = 0.0, hsum = 0.0;
  for (int e = tid; e < N; e += kFT) {
    double s = 0.0;
    int64_t cnt = 0;
#pragma unroll
    for (int h = 0; h < kFG; ++h) {
      s += gsum[h][e];
      cnt += gcnt[h][e];
    }
    const double f = (double)cnt / kl;
    lsum += f * (s / (double)L);
    if (cnt > 0) hsum -= f * log(f);
  }
  // per wave, then the wave totals in wave order
  lsum = wave_sum(lsum);
  hsum = wave_sum(hsum);
  const int wave = tid / kWave;
  if (tid % kWave == 0) {
    red[0][wave] = lsum;
    red[1][wave] = hsum;
  }
  __syncthreads();
  if (tid == 0) {
    double lt = 0.0, ht = 0.0;
    for (int w = 0; w < kFT / kWave; ++w) {
      lt += red[0][w];
      ht += red[1][w];
    }
    loss[q] = (float)(alpha * lt);
    if (entropy) entropy[q] = (float)ht;
  }
}

inline int64_t seqbal_chunks(int64_t L) { return (L + kSC - 1) / kSC; }

constexpr int64_t kMaxSeqBlocks = (int64_t)1 << 24;   // 256-thread workgroups per grid

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_seq_balance_workspace_bytes(const moe_config* cfg, int64_t T, int64_t seq_len) {
  if (check_config(cfg) != MOE_OK || T <= 0 || seq_len <= 0 || T % seq_len) return 0;
  const int64_t blocks = T / seq_len * seqbal_chunks(seq_len);
  return (size_t)blocks * cfg->n_routed * (sizeof(double) + sizeof(int32_t));
}

extern "C" moe_status moe_seq_balance(const moe_config* cfg, int64_t T, int64_t seq_len,
                                      const float* scores, const int32_t* topk_idx, float alpha,
                                      float* loss, float* entropy, void* ws, size_t ws_bytes,
                                      void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T >= ((int64_t)1 << 31) || seq_len <= 0 || T % seq_len) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!scores || !topk_idx || !loss) return MOE_ERR_NULL;
  const int64_t nseq = T / seq_len, nch = seqbal_chunks(seq_len);
  if (nseq * nch > kMaxSeqBlocks) return MOE_ERR_SHAPE;
  const int N = cfg->n_routed, k = cfg->top_k;
  const size_t need = (size_t)(nseq * nch) * N * (sizeof(double) + sizeof(int32_t));
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % alignof(double)) return MOE_ERR_UNSUPPORTED;
  double* psum = static_cast<double*>(ws);
  int32_t* pcnt = reinterpret_cast<int32_t*>(psum + nseq * nch * N);
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(seqbal_partial_kernel, dim3((unsigned)(nseq * nch)), dim3(kBT), 0, s, scores,
                     topk_idx, seq_len, nch, N, k, psum, pcnt);
  hipLaunchKernelGGL(seqbal_final_kernel, dim3((unsigned)nseq), dim3(kFT), 0, s, psum, pcnt,
                     seq_len, nch, N, k, (double)alpha, loss, entropy);
  return launch_status();
}
