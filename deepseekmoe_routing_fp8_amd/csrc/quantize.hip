// Fine-grained E4M3 quantisers: 1x128 activation tiles and 128x128 weight blocks
// (lpnh.cn guide section 3 [fp8] block; 2kiu.com digest section 4.3; zhihu infra
// commentary, per-tile 1x128 / per-group 128x128). HBM-bound: one read of the
// source, one write of codes and scales.
#include "common.h"

namespace moe {
namespace {

// 16 lanes per 128-element tile, 8 consecutive elements per lane; a 256-thread block
// covers kQTiles tiles, kQTiles/16 per thread group, with every load of a thread issued
// before the first tile is reduced. Tiles are numbered row-major over [rows, cols/128].
constexpr int kQPer = 4;
constexpr int kQTiles = 16 * kQPer;

// POW2: power-of-two group scales (scale_mode 1), for which x / s is an exact product.
template <typename T, bool POW2>
__global__ __launch_bounds__(256) void quantize_1x128_kernel(const T* __restrict__ x,
                                                             int64_t n_tiles,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scales) {
  const int sub = threadIdx.x & 15;
  float v[kQPer][8];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int64_t tile = (int64_t)blockIdx.x * kQTiles + u * 16 + (threadIdx.x >> 4);
    const int64_t base = tile * kTile + sub * 8;  // tiles are contiguous in row-major order
    if (tile < n_tiles) {
      if constexpr (sizeof(T) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[u][2 * i] = __uint_as_float(w[i] << 16);
          v[u][2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        const float4 a = *reinterpret_cast<const float4*>(x + base);
        const float4 b = *reinterpret_cast<const float4*>(x + base + 4);
        v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
        v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int64_t tile = (int64_t)blockIdx.x * kQTiles + u * 16 + (threadIdx.x >> 4);
    const int64_t base = tile * kTile + sub * 8;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
    amax = group_max<16>(amax);
    const float s = POW2 ? group_scale_pow2(amax) : group_scale(amax);
    float qv[8];
    if constexpr (POW2) {
      const float inv = inv_pow2(s);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = v[u][i] * inv;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = __fdiv_rn(v[u][i], s);
    }
    const uint32_t lo = e4m3_pack4(qv[0], qv[1], qv[2], qv[3]);
    const uint32_t hi = e4m3_pack4(qv[4], qv[5], qv[6], qv[7]);
    if (tile < n_tiles) {
      *reinterpret_cast<uint2*>(q + base) = make_uint2(lo, hi);
      if (sub == 0) scales[tile] = s;
    }
  }
}

// One 256-thread block per 128x128 block. Thread t covers rows (t/32) + 8*i, i < 16,
// and the 4 columns 4*(t%32)..+3 of each: 64 values kept in registers.
template <bool POW2>
__global__ __launch_bounds__(256) void quantize_128x128_kernel(const float* __restrict__ w,
                                                               int64_t rows, int64_t cols,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ scales) {
  const int64_t br = rows / kTile, bc = cols / kTile;
  const int64_t blk = blockIdx.x;             // (mat, block row, block col) flattened
  const int64_t mat = blk / (br * bc);
  const int64_t rem = blk % (br * bc);
  const int64_t r0 = (rem / bc) * kTile, c0 = (rem % bc) * kTile;
  const float* src = w + mat * rows * cols;
  uint8_t* dst = q + mat * rows * cols;
  const int t = threadIdx.x;
  const int rsub = t >> 5, col = (t & 31) * 4;
  float4 v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + rsub + 8 * i;
    v[i] = *reinterpret_cast<const float4*>(src + r * cols + c0 + col);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
  amax = group_max<kWave>(amax);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = POW2 ? group_scale_pow2(amax) : group_scale(amax);
  const float inv = POW2 ? inv_pow2(s) : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + rsub + 8 * i;
    const uint32_t packed =
        POW2 ? e4m3_pack4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv)
             : e4m3_pack4(__fdiv_rn(v[i].x, s), __fdiv_rn(v[i].y, s), __fdiv_rn(v[i].z, s),
                          __fdiv_rn(v[i].w, s));
    *reinterpret_cast<uint32_t*>(dst + r * cols + c0 + col) = packed;
  }
  if (t == 0) scales[blk] = s;
}

// Fragment-packed weight layout read by the grouped FFN: for a [rows, cols] matrix,
// fragment (n16, kc) = 16 rows x cols 128*kc..+127 occupies 2 KB at
// ((n16 * cols/128) + kc) * 2048, as two 1 KB halves; byte b of lane l in half h is
// W[rho(n16, l % 16)][128*kc + 64*h + 16*(l / 16) + b] with the rows of each pair of
// fragments interleaved by 4 (rho below). One thread moves 16 bytes.
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint8_t* __restrict__ q, int64_t mats,
                                                       int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit of the output
  const int64_t per_mat = rows * cols / 16;
  if (o >= mats * per_mat) return;
  const int64_t mat = o / per_mat, r = o % per_mat;
  const int lane = (int)(r & 63), half = (int)((r >> 6) & 1);
  const int64_t frag = r >> 7, nkc = cols / kTile;
  const int64_t n16 = frag / nkc, kc = frag % nkc;
  // rows of a 32-row pair of fragments interleave by 4: fragment 2m holds rows
  // 32m + 8a + b and fragment 2m+1 rows 32m + 8a + 4 + b (a, b < 4), so that the four
  // MFMA output rows a lane gets from each fragment of the pair are adjacent
  const int j = lane & 15;
  const int64_t row = 32 * (n16 >> 1) + 8 * (j >> 2) + 4 * (n16 & 1) + (j & 3);
  const int64_t col = kc * kTile + half * 64 + (lane >> 4) * 16;
  const uint4 v = *reinterpret_cast<const uint4*>(q + mat * rows * cols + row * cols + col);
  *reinterpret_cast<uint4*>(out + o * 16) = v;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_pack_fp8_weights(const uint8_t* q, int64_t mats, int64_t rows, int64_t cols,
                                           uint8_t* packed, void* stream) {
  if (mats < 0 || rows <= 0 || cols <= 0 || rows % 32 || cols % kTile) return MOE_ERR_SHAPE;
  const int64_t units = mats * rows * cols / 16;
  if (units == 0) return MOE_OK;
  if (!q || !packed) return MOE_ERR_NULL;
  if (q == packed) return MOE_ERR_UNSUPPORTED;
  const int64_t blocks = (units + 255) / 256;
  if (blocks > 0x7fffffff) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), q, mats,
                     rows, cols, packed);
  return launch_status();
}

template <bool POW2>
moe_status quantize_1x128_launch(const void* x, moe_dtype xt, int64_t rows, int64_t cols,
                                 uint8_t* q, float* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % kTile) return MOE_ERR_SHAPE;
  if (xt != MOE_F32 && xt != MOE_BF16) return MOE_ERR_DTYPE;
  const int64_t tiles = rows * (cols / kTile);
  if (tiles == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL;
  const int64_t blocks = (tiles + kQTiles - 1) / kQTiles;
  if (blocks > 0x7fffffff) return MOE_ERR_SHAPE;
  if (xt == MOE_BF16)
    hipLaunchKernelGGL((quantize_1x128_kernel<uint16_t, POW2>), dim3((unsigned)blocks), dim3(256), 0,
                       as_stream(stream), static_cast<const uint16_t*>(x), tiles, q, scales);
  else
    hipLaunchKernelGGL((quantize_1x128_kernel<float, POW2>), dim3((unsigned)blocks), dim3(256), 0,
                       as_stream(stream), static_cast<const float*>(x), tiles, q, scales);
  return launch_status();
}

template <bool POW2>
moe_status quantize_128x128_launch(const float* w, int64_t mats, int64_t rows, int64_t cols,
                                   uint8_t* q, float* scales, void* stream) {
  if (mats < 0 || rows <= 0 || cols <= 0 || rows % kTile || cols % kTile) return MOE_ERR_SHAPE;
  const int64_t blocks = mats * (rows / kTile) * (cols / kTile);
  if (blocks == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_NULL;
  if (blocks > 0x7fffffff) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(quantize_128x128_kernel<POW2>, dim3((unsigned)blocks), dim3(256), 0,
                     as_stream(stream), w, rows, cols, q, scales);
  return launch_status();
}

extern "C" moe_status moe_quantize_1x128(const void* x, moe_dtype xt, int64_t rows, int64_t cols,
                                         uint8_t* q, float* scales, void* stream) {
  return quantize_1x128_launch<false>(x, xt, rows, cols, q, scales, stream);
}

extern "C" moe_status moe_quantize_1x128_pow2(const void* x, moe_dtype xt, int64_t rows,
                                              int64_t cols, uint8_t* q, float* scales,
                                              void* stream) {
  return quantize_1x128_launch<true>(x, xt, rows, cols, q, scales, stream);
}

extern "C" moe_status moe_quantize_128x128(const float* w, int64_t mats, int64_t rows, int64_t cols,
                                           uint8_t* q, float* scales, void* stream) {
  return quantize_128x128_launch<false>(w, mats, rows, cols, q, scales, stream);
}

extern "C" moe_status moe_quantize_128x128_pow2(const float* w, int64_t mats, int64_t rows,
                                                int64_t cols, uint8_t* q, float* scales,
                                                void* stream) {
  return quantize_128x128_launch<true>(w, mats, rows, cols, q, scales, stream);
}
