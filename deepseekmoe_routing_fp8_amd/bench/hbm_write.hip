// Reference point for the write-bound kernels (the FP32 weight gradients): the store
// bandwidth this GPU reaches for the same bytes in three patterns, over a [65536, 7168]
// float matrix (1.75 GiB):
//   linear    16-byte stores, grid-stride over the whole buffer;
//   wgrad     the weight-gradient kernel's pattern: a 256-thread workgroup writes a
//             128 x 128 tile, each wave a 64 x 64 quarter, each store instruction 16 rows
//             x 64 contiguous bytes (lane l: row l % 16, 16 bytes at column 4 (l / 16));
//   rows      the same tiles written as two 512-byte row pieces per store instruction;
//   pairs     the gate/up epilogue's pattern for its FP32 rows: a 512-thread workgroup
//             writes 16 rows x 128 columns per step, wave w lane l 16 bytes at row l % 16,
//             column 32 (w / 2) + 8 (l / 16) + 4 (w % 2), so the two halves of every
//             32-byte piece come from two waves.
// Prints the best time of three per pattern (event-timed).
#include <hip/hip_runtime.h>

#include <cstdio>

typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kR = 65536, kC = 7168;

__global__ __launch_bounds__(256) void store_linear(float* __restrict__ out, long n4, float v) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256)
    reinterpret_cast<v4f*>(out)[i] = v4f{v, v, v, v};
}

__global__ __launch_bounds__(256) void store_wgrad(float* __restrict__ out, float v) {
  const int tc = blockIdx.x % (kC / 128), tr = blockIdx.x / (kC / 128);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const int wn = tr * 128 + (wave >> 1) * 64, wm = tc * 128 + (wave & 1) * 64;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<v4f*>(out + (long)(wn + 16 * i + lr) * kC + wm + 16 * j + 4 * lg) = v4f{v, v, v, v};
}

__global__ __launch_bounds__(256) void store_rows(float* __restrict__ out, float v) {
  const int tc = blockIdx.x % (kC / 128), tr = blockIdx.x / (kC / 128);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = 0; i < 16; ++i) {
    const int row = tr * 128 + wave * 32 + 2 * i + (lane >> 5);
    *reinterpret_cast<v4f*>(out + (long)row * kC + tc * 128 + 4 * (lane & 31)) = v4f{v, v, v, v};
  }
}

__global__ __launch_bounds__(512) void store_pairs(float* __restrict__ out, float v) {
  const int tc = blockIdx.x % (kC / 128), tr = blockIdx.x / (kC / 128);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = tc * 128 + 32 * (wave >> 1) + 8 * (lane >> 4) + 4 * (wave & 1);
  for (int ts = 0; ts < 8; ++ts)   // 128 rows per workgroup
    *reinterpret_cast<v4f*>(out + (long)(tr * 128 + ts * 16 + (lane & 15)) * kC + col) = v4f{v, v, v, v};
}

int main() {
  const size_t bytes = (size_t)kR * kC * 4;
  float* out = nullptr;
  if (hipMalloc(&out, bytes) != hipSuccess) {
    std::printf("allocation failed\n");
    return 1;
  }
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  const int tiles = (kR / 128) * (kC / 128);
  const char* names[4] = {"linear", "wgrad 16 rows x 64 B", "rows 2 x 512 B", "pairs 16 B halves"};
  for (int k = 0; k < 4; ++k) {
    float best = 1e30f;
    for (int r = 0; r < 4; ++r) {   // the first run of each pattern is a warm-up
      hipEventRecord(a);
      if (k == 0) hipLaunchKernelGGL(store_linear, dim3(4096), dim3(256), 0, 0, out, (long)(bytes / 16), 1.0f);
      if (k == 1) hipLaunchKernelGGL(store_wgrad, dim3(tiles), dim3(256), 0, 0, out, 2.0f);
      if (k == 2) hipLaunchKernelGGL(store_rows, dim3(tiles), dim3(256), 0, 0, out, 3.0f);
      if (k == 3) hipLaunchKernelGGL(store_pairs, dim3(tiles), dim3(512), 0, 0, out, 4.0f);
      hipEventRecord(b);
      if (hipEventSynchronize(b) != hipSuccess) return 1;
      float ms = 0.0f;
      hipEventElapsedTime(&ms, a, b);
      if (r > 0) best = ms < best ? ms : best;
    }
    std::printf("%-22s %.3f ms, %.2f TB/s\n", names[k], best, bytes / (best * 1e-3) / 1e12);
  }
  hipFree(out);
  return 0;
}
