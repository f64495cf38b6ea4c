// Weighted combine and sign-based bias update.
//   combine: 2kiu.com digest section 3.2 (y = sum_j gate[j] * ffn_expert[idx[j]](h)) plus
//   the shared experts with gate 1 (lpnh.cn guide section 3: num_shared_experts).
//   bias update: same digest, section 3.2 pseudocode (after a step, over-loaded experts
//   lose gamma, under-loaded ones gain gamma) and section 5.2 (whole-batch statistics).
#include "common.h"

namespace moe {
namespace {

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float (&v)[8]) {
  if constexpr (sizeof(YT) == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename YT>
__device__ __forceinline__ void unpack8(const uint4 (&raw)[sizeof(YT) / 2], float (&v)[8]) {
  if constexpr (sizeof(YT) == 2) {
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(raw[0].x); v[1] = __uint_as_float(raw[0].y);
    v[2] = __uint_as_float(raw[0].z); v[3] = __uint_as_float(raw[0].w);
    v[4] = __uint_as_float(raw[1].x); v[5] = __uint_as_float(raw[1].y);
    v[6] = __uint_as_float(raw[1].z); v[7] = __uint_as_float(raw[1].w);
  }
}

// One block per token; each thread sums 8 consecutive features per step, in the fixed
// order: shared experts 0..N_s-1, then slots 0..k-1 (FP32), then one rounding to bf16.
// All slots' rows of a step are loaded before any is added (a skipped slot reads row 0
// and contributes exactly zero), so the loads of one step are in flight together.
template <typename YT>
__global__ __launch_bounds__(1024) void combine_kernel(const YT* __restrict__ y_rows,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      const YT* __restrict__ y_shared, int n_shared,
                                                      int64_t T, int H, int k, int64_t n_rows,
                                                      uint16_t* __restrict__ out) {
  constexpr int U = sizeof(YT) / 2;   // 16-byte units per 8 values
  const int64_t t = blockIdx.x;
  __shared__ int32_t rows[kMaxTopK];
  __shared__ float g[kMaxTopK];
  if (threadIdx.x < kMaxTopK) {
    int32_t r = -1;
    float gv = 0.0f;
    if (threadIdx.x < k) {
      r = row_of[t * k + threadIdx.x];
      gv = gate[t * k + threadIdx.x];
    }
    rows[threadIdx.x] = (r >= 0 && r < n_rows) ? r : -1;
    g[threadIdx.x] = gv;
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sidx = 0; sidx < n_shared; ++sidx) {
      float v[8];
      load8(y_shared + ((int64_t)sidx * T + t) * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    uint4 raw[kMaxTopK][U];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const YT* p = y_rows + (int64_t)max(rows[j], 0) * H + c;
#pragma unroll
        for (int u = 0; u < U; ++u) raw[j][u] = reinterpret_cast<const uint4*>(p)[u];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && rows[j] >= 0) {
        float v[8];
        unpack8<YT>(raw[j], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[i], acc[i]);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
}

__global__ void update_bias_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                   int N, int64_t target_num, float gamma) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N) return;
  // target load T*k/N compared as T*k vs N*count, in integers
  const int64_t lhs = target_num, rhs = (int64_t)N * counts[e];
  const float d = lhs > rhs ? gamma : (lhs < rhs ? -gamma : 0.0f);
  bias[e] = bias[e] + d;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, moe_dtype yt,
                                  const int32_t* row_of, const float* topk_gate, const void* y_shared,
                                  uint16_t* out, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > 0x7fffffff) return MOE_ERR_SHAPE;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!y_rows || !row_of || !topk_gate || !out) return MOE_ERR_NULL;
  if (cfg->n_shared > 0 && !y_shared) return MOE_ERR_NULL;
  const int64_t n_rows = T * cfg->top_k;
  hipStream_t s = as_stream(stream);
  // Few tokens (fewer blocks than a few per CU): one thread per 16-byte step of the row,
  // every load of the token in flight at once (V3 decode, T = 128: 8 against 15 us).
  // Many tokens: 256 threads, several steps each (at T = 4096, 896 threads measured 16%
  // slower and 128 threads 15% slower).
  const int units = cfg->hidden / 8;
  const int nthr = T < 2048 && units <= 1024 ? (units + 63) / 64 * 64 : 256;
  if (yt == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((unsigned)T), dim3(nthr), 0, s,
                       static_cast<const uint16_t*>(y_rows), row_of, topk_gate,
                       static_cast<const uint16_t*>(y_shared), cfg->n_shared, T, cfg->hidden,
                       cfg->top_k, n_rows, out);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)T), dim3(nthr), 0, s,
                       static_cast<const float*>(y_rows), row_of, topk_gate,
                       static_cast<const float*>(y_shared), cfg->n_shared, T, cfg->hidden,
                       cfg->top_k, n_rows, out);
  return launch_status();
}

extern "C" moe_status moe_update_bias(const moe_config* cfg, int64_t T, const int32_t* counts,
                                      float* bias, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return MOE_ERR_NULL;
  if (T < 0 || T > ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  const int N = cfg->n_routed;
  hipLaunchKernelGGL(update_bias_kernel, dim3((N + 255) / 256), dim3(256), 0, as_stream(stream),
                     counts, bias, N, T * cfg->top_k, cfg->bias_gamma);
  return launch_status();
}

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size or configuration field is out of range";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_UNSUPPORTED: return "unsupported request";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_SCRATCH:
      return "the request needs more workspace than the library's static scratch buffer holds";
  }
  return "unknown status";
}
