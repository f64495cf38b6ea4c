// Reference point for the HBM rooflines: the read bandwidth a plain streaming kernel
// reaches on this GPU. Reads an 8 GiB buffer with 16-byte loads over grid sizes from
// 1024 to 8192 workgroups of 256 threads, and prints the best time of three per size.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdint>

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n,
                                                   unsigned* __restrict__ out) {
  unsigned acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;   // keeps the loads; practically never taken
}

int main() {
  const size_t bytes = (size_t)8 << 30, n = bytes / 16;
  uint4* p = nullptr;
  unsigned* o = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || hipMalloc(&o, 4) != hipSuccess) {
    std::printf("allocation failed\n");
    return 1;
  }
  if (hipMemset(p, 1, bytes) != hipSuccess) return 1;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  float best_all = 1e30f;
  for (int g : {1024, 2048, 4096, 8192}) {
    float best = 1e30f;
    for (int r = 0; r < 3; ++r) {
      hipEventRecord(a);
      hipLaunchKernelGGL(stream_read, dim3(g), dim3(256), 0, 0, p, n, o);
      hipEventRecord(b);
      hipEventSynchronize(b);
      float ms = 0.0f;
      hipEventElapsedTime(&ms, a, b);
      best = ms < best ? ms : best;
    }
    best_all = best < best_all ? best : best_all;
    std::printf("grid %d: %.3f ms, %.2f TB/s\n", g, best, bytes / (best * 1e-3) / 1e12);
  }
  std::printf("best: %.2f TB/s (%.1f%% of 8 TB/s)\n", bytes / (best_all * 1e-3) / 1e12,
              bytes / (best_all * 1e-3) / 1e12 / 8.0 * 100.0);
  hipFree(p);
  hipFree(o);
  return 0;
}
