// Native driver of one MoE-layer step for hardware-counter runs: the six C entry points
// (moe_quantize_1x128, moe_route, moe_permute, moe_grouped_ffn_fp8_gate_up / _down,
// moe_combine, moe_update_bias) at the DeepSeek-V3 shape (H = 7168, I = 2048, 256 routed
// experts in 8 groups of 32, keep 4, top-8, 1 shared expert), without Python, so that a
// profiler session sees only these launches.
//
// Workloads: prefill (T = 4096), decode (T = 128), skewed (T = 16384, tokens drawn from 64
// Gaussian clusters with Zipf(1.1) frequencies whose centroids are 2 x the unit router
// rows of 64 seeded experts). Weights are N(0, 1/fan_in), quantised to E4M3 128x128 blocks
// and packed on the device by the library itself; x is N(0, 1) (plus the centroid) in
// bf16. The generators are counter-based hashes (splitmix64 + Box-Muller): the same
// shapes and distributions as the test inputs, not the same values.
//
// A plain copy kernel over a buffer of known size runs first; its counter readings
// calibrate the byte counters.
//
// Usage: moe_counters <prefill|decode|skewed> [reps=3] [copy_mib=2048]
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe_fp8.h"

#define CK(x)                                                                             \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)
#define CM(x)                                                                         \
  do {                                                                                \
    moe_status s_ = (x);                                                              \
    if (s_ != MOE_OK) {                                                               \
      std::fprintf(stderr, "%s at line %d\n", moe_status_string(s_), __LINE__);       \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__host__ __device__ inline uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// N(0, 1) from the counter (seed, i) by Box-Muller on two 32-bit uniforms.
__host__ __device__ inline float gauss(uint64_t seed, uint64_t i) {
  const uint64_t h = splitmix64(seed * 0xD1B54A32D192ED03ull + i);
  const float u1 = ((uint32_t)h + 1.0f) * 2.3283064365386963e-10f;   // (0, 1]
  const float u2 = (uint32_t)(h >> 32) * 2.3283064365386963e-10f;
  return sqrtf(-2.0f * logf(u1)) * cosf(6.283185307179586f * u2);
}

__global__ void fill_gauss(float* p, size_t n, uint64_t seed, float sd) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = sd * gauss(seed, i);
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// x[t, h] = centroid (2 x unit router row of the token's cluster, or 0) + N(0, 1), as bf16
__global__ void fill_x(uint16_t* x, int T, int H, const float* __restrict__ wr,
                       const int32_t* __restrict__ cent_row, const float* __restrict__ cent_scale,
                       uint64_t seed) {
  const size_t n = (size_t)T * H;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / H), h = (int)(i % H);
    float v = gauss(seed, i);
    if (cent_row) v += cent_scale[t] * wr[(size_t)cent_row[t] * H + h];
    x[i] = bf16_rne(v);
  }
}

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s <prefill|decode|skewed> [reps] [copy_mib]\n", argv[0]);
    return 2;
  }
  const std::string wl = argv[1];
  const int reps = argc > 2 ? std::atoi(argv[2]) : 3;
  const size_t copy_bytes = (size_t)(argc > 3 ? std::atoi(argv[3]) : 2048) << 20;
  int T;
  if (wl == "prefill") T = 4096;
  else if (wl == "decode") T = 128;
  else if (wl == "skewed") T = 16384;
  else {
    std::fprintf(stderr, "unknown workload %s\n", wl.c_str());
    return 2;
  }
  const int H = 7168, I = 2048, NR = 256, NS = 1, K = 8;
  const int EA = NR + NS;
  const int64_t rows = (int64_t)T * (K + NS);
  moe_config c{H, I, NR, NS, K, 8, 4, 2, 2.5f, 0.001f, 0};

  // copy calibration
  uint4 *csrc, *cdst;
  CK(hipMalloc(&csrc, copy_bytes));
  CK(hipMalloc(&cdst, copy_bytes));
  hipLaunchKernelGGL(fill_gauss, dim3(4096), dim3(256), 0, nullptr, (float*)csrc, copy_bytes / 4, 9, 1.0f);
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

  // router weight (host, so that its row norms give the cluster centroids) and its planes
  std::vector<float> wr_h((size_t)NR * H);
  for (size_t i = 0; i < wr_h.size(); ++i) wr_h[i] = gauss(11, i) / std::sqrt((float)H);
  float* wr;
  CK(hipMalloc(&wr, wr_h.size() * 4));
  CK(hipMemcpy(wr, wr_h.data(), wr_h.size() * 4, hipMemcpyHostToDevice));
  uint16_t* wsplit;
  CK(hipMalloc(&wsplit, moe_router_weights_elems(NR, H) * 2));
  CM(moe_pack_router_weights(wr, NR, H, wsplit, nullptr));

  // experts: N(0, 1/fan_in) -> 128x128 E4M3 blocks -> packed, one matrix at a time
  uint8_t *w1, *w3, *w2, *tmpq;
  float *w1s, *w3s, *w2s, *tmpf;
  const size_t mat = (size_t)I * H, nsc = (size_t)(I / 128) * (H / 128);
  CK(hipMalloc(&w1, EA * mat));
  CK(hipMalloc(&w3, EA * mat));
  CK(hipMalloc(&w2, EA * mat));
  CK(hipMalloc(&w1s, EA * nsc * 4));
  CK(hipMalloc(&w3s, EA * nsc * 4));
  CK(hipMalloc(&w2s, EA * nsc * 4));
  CK(hipMalloc(&tmpq, mat));
  CK(hipMalloc(&tmpf, mat * 4));
  for (int e = 0; e < EA; ++e) {
    for (int m = 0; m < 3; ++m) {
      const bool down = m == 2;
      hipLaunchKernelGGL(fill_gauss, dim3(2048), dim3(256), 0, nullptr, tmpf, mat,
                         (uint64_t)(100 + 3 * e + m), 1.0f / std::sqrt((float)(down ? I : H)));
      uint8_t* q = (m == 0 ? w1 : m == 1 ? w3 : w2) + (size_t)e * mat;
      float* s = (m == 0 ? w1s : m == 1 ? w3s : w2s) + (size_t)e * nsc;
      CM(moe_quantize_128x128(tmpf, 1, down ? H : I, down ? I : H, tmpq, s, nullptr));
      CM(moe_pack_fp8_weights(tmpq, 1, down ? H : I, down ? I : H, q, nullptr));
    }
  }
  CK(hipFree(tmpq));
  CK(hipFree(tmpf));

  // hidden states
  uint16_t* x;
  CK(hipMalloc(&x, (size_t)T * H * 2));
  int32_t* cent_row = nullptr;
  float* cent_scale = nullptr;
  if (wl == "skewed") {
    // 64 clusters, P(j) ~ j^-1.1; centroid j = 2 x unit row of expert perm[j]
    std::vector<double> cdf(64);
    double z = 0;
    for (int j = 0; j < 64; ++j) cdf[j] = (z += std::pow(j + 1.0, -1.1));
    std::vector<int> perm(NR);
    for (int i = 0; i < NR; ++i) perm[i] = i;
    uint64_t st = 77;
    for (int i = NR - 1; i > 0; --i) std::swap(perm[i], perm[splitmix64(st++) % (i + 1)]);
    std::vector<int32_t> rowv(T);
    std::vector<float> scv(T);
    for (int t = 0; t < T; ++t) {
      const double u = (splitmix64(1000 + t) >> 11) * (1.0 / 9007199254740992.0) * z;
      int j = 0;
      while (j < 63 && cdf[j] < u) ++j;
      const int e = perm[j];
      double nn = 0;
      for (int h = 0; h < H; ++h) nn += (double)wr_h[(size_t)e * H + h] * wr_h[(size_t)e * H + h];
      rowv[t] = e;
      scv[t] = (float)(2.0 / std::sqrt(nn));
    }
    CK(hipMalloc(&cent_row, T * 4));
    CK(hipMalloc(&cent_scale, T * 4));
    CK(hipMemcpy(cent_row, rowv.data(), T * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(cent_scale, scv.data(), T * 4, hipMemcpyHostToDevice));
  }
  hipLaunchKernelGGL(fill_x, dim3(2048), dim3(256), 0, nullptr, x, T, H, wr, cent_row, cent_scale, 5);

  // step buffers
  uint8_t* xq;
  float *xs, *bias, *scores, *gate;
  int32_t *idx, *counts, *offsets, *row_token, *row_of;
  uint16_t *y, *out;
  CK(hipMalloc(&xq, (size_t)T * H));
  CK(hipMalloc(&xs, (size_t)T * (H / 128) * 4));
  CK(hipMalloc(&bias, NR * 4));
  CK(hipMalloc(&scores, (size_t)T * NR * 4));
  CK(hipMalloc(&gate, (size_t)T * K * 4));
  CK(hipMalloc(&idx, (size_t)T * K * 4));
  CK(hipMalloc(&counts, NR * 4));
  CK(hipMalloc(&offsets, (EA + 1) * 4));
  CK(hipMalloc(&row_token, rows * 4));
  CK(hipMalloc(&row_of, (size_t)T * K * 4));
  CK(hipMalloc(&y, (size_t)rows * H * 2));
  CK(hipMalloc(&out, (size_t)T * H * 2));
  const size_t rwsn = moe_route_workspace_bytes(&c, T, MOE_BF16);
  const size_t pwsn = moe_permute_workspace_bytes(&c, T);
  const size_t fwsn = moe_grouped_ffn_workspace_bytes(&c, EA, rows);
  void *rws, *pws, *fws;
  CK(hipMalloc(&rws, rwsn > 0 ? rwsn : 1));
  CK(hipMalloc(&pws, pwsn > 0 ? pwsn : 1));
  CK(hipMalloc(&fws, fwsn));
  CK(hipDeviceSynchronize());

  const char* names[] = {"quantize", "route", "permute", "gate_up", "down", "combine", "bias_update"};
  constexpr int NS_ = 7;
  std::vector<hipEvent_t> ev((NS_ + 1) * reps);
  for (auto& e : ev) CK(hipEventCreate(&e));
  std::vector<int32_t> load(NR);
  for (int r = 0; r < reps; ++r) {
    CK(hipMemset(bias, 0, NR * 4));   // the configured bias (zeros) at every repetition
    hipEvent_t* E = &ev[(NS_ + 1) * r];
    CK(hipEventRecord(E[0]));
    CM(moe_quantize_1x128(x, MOE_BF16, T, H, xq, xs, nullptr));
    CK(hipEventRecord(E[1]));
    CM(moe_route(&c, x, MOE_BF16, T, wsplit, bias, scores, idx, gate, counts, rws, rwsn, nullptr));
    CK(hipEventRecord(E[2]));
    CM(moe_permute(&c, T, idx, offsets, row_token, row_of, pws, pwsn, nullptr));
    CK(hipEventRecord(E[3]));
    CM(moe_grouped_ffn_fp8_gate_up(&c, EA, rows, T, xq, xs, row_token, offsets, w1, w1s, w3, w3s,
                                   fws, fwsn, nullptr));
    CK(hipEventRecord(E[4]));
    CM(moe_grouped_ffn_fp8_down(&c, EA, rows, w2, w2s, y, MOE_BF16, fws, fwsn, nullptr));
    CK(hipEventRecord(E[5]));
    CM(moe_combine(&c, T, y, MOE_BF16, row_of, gate, y + (size_t)T * K * H, out, nullptr));
    CK(hipEventRecord(E[6]));
    CM(moe_update_bias(&c, T, counts, bias, nullptr));
    CK(hipEventRecord(E[7]));
  }
  CK(hipDeviceSynchronize());
  CK(hipMemcpy(load.data(), counts, NR * 4, hipMemcpyDeviceToHost));
  int mx = 0, touched = 0;
  for (int v : load) {
    mx = v > mx ? v : mx;
    touched += v > 0;
  }
  std::printf("workload %s: T=%d H=%d I=%d routed=%d shared=%d top_k=%d rows=%lld; experts touched "
              "%d, max/mean load %.3f\n",
              wl.c_str(), T, H, I, NR, NS, K, (long long)rows, touched, mx / (double)(T * K / NR));
  for (int s = 0; s < NS_; ++s) {
    double sum = 0;
    for (int r = 0; r < reps; ++r) {
      float a = 0;
      CK(hipEventElapsedTime(&a, ev[(NS_ + 1) * r + s], ev[(NS_ + 1) * r + s + 1]));
      sum += a;
    }
    std::printf("  %-12s %.4f ms per call (%d calls)\n", names[s], sum / reps, reps);
  }
  std::printf("expert loads:");
  for (int v : load) std::printf(" %d", v);
  std::printf("\n");
  return 0;
}
