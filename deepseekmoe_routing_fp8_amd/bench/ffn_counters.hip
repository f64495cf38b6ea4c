// Native driver for hardware-counter runs of the grouped FP8 FFN at the DeepSeek-V3
// prefill shape: T = 4096 tokens, H = 7168, I = 2048, 256 routed experts + 1 shared,
// top-8 routing. Runs without Python so that a profiler session sees only these launches.
//
// It first runs a plain copy kernel over a buffer of known size, whose counter readings
// calibrate the byte counters, then `reps` calls of moe_grouped_ffn_fp8_gate_up and
// moe_grouped_ffn_fp8_down through the C ABI (routing and permutation by moe_permute on
// seeded uniform top-8 choices; codes and scales are seeded random bytes, which leaves
// the data movement of the kernels unchanged).
//
// Usage: ffn_counters [reps=5] [copy_mib=2048]
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/moe_fp8.h"

#define CK(x)                                                                       \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                     \
    }                                                                               \
  } while (0)
#define CM(x)                                                                       \
  do {                                                                              \
    moe_status s_ = (x);                                                            \
    if (s_ != MOE_OK) {                                                             \
      std::fprintf(stderr, "%s at line %d\n", moe_status_string(s_), __LINE__);     \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__device__ uint32_t mix32(uint64_t v) {
  v ^= v >> 33;
  v *= 0xff51afd7ed558ccdull;
  v ^= v >> 33;
  v *= 0xc4ceb9fe1a85ec53ull;
  v ^= v >> 33;
  return (uint32_t)v;
}

// E4M3 codes without the NaN patterns 0x7F / 0xFF
__global__ void fill_codes(uint8_t* p, size_t n, uint64_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint32_t h = mix32(seed * 0x9E3779B97F4A7C15ull + i);
    p[i] = (uint8_t)((h % 0x7F) | ((h >> 8) & 0x80));
  }
}

__global__ void fill_scales(float* p, size_t n, uint64_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = (0.5f + (mix32(seed * 0x9E3779B97F4A7C15ull + i) & 0xFFFF) / 65536.0f) / 448.0f;
}

static uint64_t splitmix(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main(int argc, char** argv) {
  const int reps = argc > 1 ? std::atoi(argv[1]) : 5;
  const size_t copy_bytes = (size_t)(argc > 2 ? std::atoi(argv[2]) : 2048) << 20;
  const int T = 4096, H = 7168, I = 2048, NR = 256, NS = 1, K = 8;
  const int EA = NR + NS;
  const int64_t rows = (int64_t)T * (K + NS);
  moe_config c{H, I, NR, NS, K, 8, 4, 2, 2.5f, 0.001f};

  // copy calibration
  uint4 *csrc, *cdst;
  CK(hipMalloc(&csrc, copy_bytes));
  CK(hipMalloc(&cdst, copy_bytes));
  hipLaunchKernelGGL(fill_codes, dim3(4096), dim3(256), 0, nullptr, (uint8_t*)csrc, copy_bytes, 9);
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(copy_kernel, dim3(8192), dim3(256), 0, nullptr, csrc, cdst, copy_bytes / 16);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms = 0;
  CK(hipEventElapsedTime(&ms, e0, e1));
  std::printf("copy_kernel: %zu bytes read + %zu bytes written in %.3f ms (%.0f GB/s)\n",
              copy_bytes, copy_bytes, ms, 2.0 * copy_bytes / ms / 1e6);
  CK(hipFree(csrc));
  CK(hipFree(cdst));

  // inputs
  uint8_t *xq, *w1, *w3, *w2;
  float *xs, *w1s, *w3s, *w2s;
  const size_t wbytes = (size_t)EA * I * H, sbytes = (size_t)EA * (I / 128) * (H / 128);
  CK(hipMalloc(&xq, (size_t)T * H));
  CK(hipMalloc(&xs, (size_t)T * (H / 128) * 4));
  CK(hipMalloc(&w1, wbytes));
  CK(hipMalloc(&w3, wbytes));
  CK(hipMalloc(&w2, wbytes));
  CK(hipMalloc(&w1s, sbytes * 4));
  CK(hipMalloc(&w3s, sbytes * 4));
  CK(hipMalloc(&w2s, sbytes * 4));
  hipLaunchKernelGGL(fill_codes, dim3(4096), dim3(256), 0, nullptr, xq, (size_t)T * H, 1);
  hipLaunchKernelGGL(fill_codes, dim3(4096), dim3(256), 0, nullptr, w1, wbytes, 2);
  hipLaunchKernelGGL(fill_codes, dim3(4096), dim3(256), 0, nullptr, w3, wbytes, 3);
  hipLaunchKernelGGL(fill_codes, dim3(4096), dim3(256), 0, nullptr, w2, wbytes, 4);
  hipLaunchKernelGGL(fill_scales, dim3(256), dim3(256), 0, nullptr, xs, (size_t)T * (H / 128), 5);
  hipLaunchKernelGGL(fill_scales, dim3(256), dim3(256), 0, nullptr, w1s, sbytes, 6);
  hipLaunchKernelGGL(fill_scales, dim3(256), dim3(256), 0, nullptr, w3s, sbytes, 7);
  hipLaunchKernelGGL(fill_scales, dim3(256), dim3(256), 0, nullptr, w2s, sbytes, 8);

  // seeded uniform top-8 choices (distinct experts per token), then the real permutation
  std::vector<int32_t> idx((size_t)T * K);
  uint64_t st = 12345;
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K;) {
      const int e = (int)(splitmix(st) % NR);
      bool dup = false;
      for (int i = 0; i < j; ++i) dup |= idx[(size_t)t * K + i] == e;
      if (!dup) idx[(size_t)t * K + j++] = e;
    }
  }
  int32_t *d_idx, *offsets, *row_token, *row_of;
  CK(hipMalloc(&d_idx, idx.size() * 4));
  CK(hipMalloc(&offsets, (EA + 1) * 4));
  CK(hipMalloc(&row_token, rows * 4));
  CK(hipMalloc(&row_of, (size_t)T * K * 4));
  CK(hipMemcpy(d_idx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
  void* pws;
  const size_t pwsn = moe_permute_workspace_bytes(&c, T);
  CK(hipMalloc(&pws, pwsn));
  CM(moe_permute(&c, T, d_idx, offsets, row_token, row_of, pws, pwsn, nullptr));

  uint16_t* y;
  CK(hipMalloc(&y, (size_t)rows * H * 2));
  const size_t wsn = moe_grouped_ffn_workspace_bytes(&c, EA, rows);
  void* ws;
  CK(hipMalloc(&ws, wsn));
  CK(hipDeviceSynchronize());

  std::vector<hipEvent_t> ev(3 * reps);
  for (auto& e : ev) CK(hipEventCreate(&e));
  for (int r = 0; r < reps; ++r) {
    CK(hipEventRecord(ev[3 * r]));
    CM(moe_grouped_ffn_fp8_gate_up(&c, EA, rows, T, xq, xs, row_token, offsets, w1, w1s, w3, w3s,
                                   ws, wsn, nullptr));
    CK(hipEventRecord(ev[3 * r + 1]));
    CM(moe_grouped_ffn_fp8_down(&c, EA, rows, w2, w2s, y, MOE_BF16, ws, wsn, nullptr));
    CK(hipEventRecord(ev[3 * r + 2]));
  }
  CK(hipDeviceSynchronize());
  double gu = 0, dn = 0;
  for (int r = 0; r < reps; ++r) {
    float a = 0, b = 0;
    CK(hipEventElapsedTime(&a, ev[3 * r], ev[3 * r + 1]));
    CK(hipEventElapsedTime(&b, ev[3 * r + 1], ev[3 * r + 2]));
    gu += a;
    dn += b;
  }
  std::printf("moe_grouped_ffn_fp8_gate_up: %.4f ms per call (%d calls, incl. tile plan)\n",
              gu / reps, reps);
  std::printf("moe_grouped_ffn_fp8_down:    %.4f ms per call\n", dn / reps);
  std::printf("shape: T=%d H=%d I=%d routed=%d shared=%d top_k=%d rows=%lld\n", T, H, I, NR, NS, K,
              (long long)rows);
  return 0;
}
