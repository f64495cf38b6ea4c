// Backward pass of the DeepSeekMoE layer with FP8 GEMMs.
//
// Sources, by page and section:
//   lpnh.cn guide "从技术报告到可跑配置", section 3: the [fp8] block runs fprop, dgrad and
//   wgrad GEMMs in FP8 e4m3 with 1x128 tile-wise inputs and 128x128 block-wise weights,
//   and keeps moe_gating in BF16/FP32;
//   zhihu infra commentary, training part: E4M3 in both directions, per-tile and
//   per-group scaling, GEMMs by partial-sum promotion, SwiGLU recomputed;
//   2kiu.com digest, section 3.2: gates are the normalised unbiased affinities of the
//   selected experts times the scaling factor.
//
// Steps and launches:
//   combine backward   the gates' gradient (dot products) and each row's gate (dy of a row,
//                      gate x dout, is formed where the FFN backward quantises it);
//   router backward    gate gradient -> affinity -> logit gradient (FP32), then dx of the
//                      router GEMM and dW_r summed per expert in segment order;
//   FFN backward       per expert segment, on the forward's tile plan:
//     dy = gate x dout -> 1x128 along H     (dgrad operand)
//     a = xq W1^T, b = xq W3^T              (the SwiGLU inputs: kept by a training forward,
//                                            else recomputed by the gate/up launch, FP32)
//     dh = dy W2                            (FP8 grouped GEMM, K = H, FP32 out)
//     dg, du, h (FP32) -> [dg | du] 1x128 along I   (dgrad operand, K = 2I)
//     dx_rows = [dg | du] [W1 ; W3]         (one FP8 grouped GEMM on [W1^T | W3^T])
//     dy, h, dg, du, x  -> 128-row tiles along the token axis, stored transposed
//     dW2 = dy^T h; dW1 = dg^T x and dW3 = du^T x in one launch   (FP8 wgrad, K = tokens)
//   unpermute-sum      dx_t = sum of its rows' dx (+ the router's dx), FP32, bf16 out.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "ffn_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 8 consecutive values at p[i..i+8) (i a multiple of 8) as floats.
template <typename T>
__device__ __forceinline__ void ld8(const T* p, int64_t i, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Sum over the 256 threads of a block, one value per slot (k <= kMaxTopK slots), in a fixed
// order: lanes by butterfly, then the four waves in order.
__device__ __forceinline__ void block_sum_slots(float (&v)[kMaxTopK], int k, float* red,
                                                float* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int j = 0; j < k; ++j) {
    float x = v[j];
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, kWave);
    if (lane == 0) red[wave * kMaxTopK + j] = x;
  }
  __syncthreads();
  if (tid < k) out[tid] = ((red[tid] + red[kMaxTopK + tid]) + red[2 * kMaxTopK + tid]) + red[3 * kMaxTopK + tid];
}

// ------------------------------------------------------------------------------------
// Combine backward: one block per token. The rows' upstream gradient dy_r = gate_r dout_t is
// not materialised: the block writes the gate of each of the token's rows (1 for the
// shared rows), and the FFN backward forms the product where it quantises dy.
// ------------------------------------------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dout,
                                                          const YT* __restrict__ y_rows,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ gate,
                                                          int64_t T, int H, int k, int S,
                                                          int64_t n_rows, float* __restrict__ row_gate,
                                                          float* __restrict__ dgate) {
  __shared__ int32_t rows[kMaxTopK];
  __shared__ float g[kMaxTopK];
  __shared__ float red[4 * kMaxTopK];
  __shared__ float res[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < kMaxTopK) {
    int32_t r = -1;
    float gv = 0.0f;
    if (threadIdx.x < k) {
      r = row_of[t * k + threadIdx.x];
      gv = gate[t * k + threadIdx.x];
    }
    r = (r >= 0 && r < n_rows) ? r : -1;
    rows[threadIdx.x] = r;
    g[threadIdx.x] = gv;
    if (r >= 0) row_gate[r] = gv;
  } else if (threadIdx.x < kMaxTopK + S) {
    row_gate[T * k + (threadIdx.x - kMaxTopK) * T + t] = 1.0f;
  }
  __syncthreads();
  float part[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) part[j] = 0.0f;
  // 8 consecutive features per thread and step; every slot's row is read before any is
  // used, so a step's loads are in flight together
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float d[8];
    ld8(dout, t * H + c, d);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && rows[j] >= 0) {
        float y[8];
        ld8(y_rows, (int64_t)rows[j] * H + c, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) part[j] = fmaf(d[i], y[i], part[j]);
      }
    }
  }
  block_sum_slots(part, k, red, res);
  if (threadIdx.x < k) dgate[t * k + threadIdx.x] = rows[threadIdx.x] >= 0 ? res[threadIdx.x] : 0.0f;
}

// ------------------------------------------------------------------------------------
// Router backward.
//   gates:  per token, for the k selected experts: ds_m = (rho / Z)(dg_m - sum_j dg_j g_j / rho),
//           Z = sum of the selected s; dlogit = ds s (1 - s). Also scattered per permuted row.
//   dx:     dx_t = sum_j dlogit_tj W_r[e_j]               (one block per token)
//   dw:     dW_r[e] = sum over e's rows r of dlogit_r x_{token(r)}, in row order
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_bwd_gates_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ idx,
                                                              const float* __restrict__ dgate,
                                                              const int32_t* __restrict__ row_of,
                                                              int64_t T, int N, int k, float rho,
                                                              int64_t n_rows,
                                                              float* __restrict__ dl,
                                                              float* __restrict__ dl_row) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float s[kMaxTopK], dg[kMaxTopK];
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    s[j] = 0.0f;
    dg[j] = 0.0f;
    if (j < k) {
      const int e = idx[t * k + j];
      s[j] = (e >= 0 && e < N) ? scores[t * N + e] : 0.0f;
      dg[j] = dgate[t * k + j];
      z += s[j];
    }
  }
  // sum_j dg_j g_j / rho = sum_j dg_j s_j / Z
  float inner = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) inner = fmaf(dg[j], s[j], inner);
  inner = z > 0.0f ? inner / z : 0.0f;
  const float f = z > 0.0f ? rho / z : 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      const float v = f * (dg[j] - inner) * s[j] * (1.0f - s[j]);
      dl[t * k + j] = v;
      const int32_t r = row_of[t * k + j];
      if (r >= 0 && r < n_rows) dl_row[r] = v;
    }
  }
}

// dx: one block per token, four consecutive features per thread and step; every slot's
// row of W_r is loaded before any is added, and the slots are added in order.
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(const float* __restrict__ dl,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ w_router,
                                                           int N, int k, int H,
                                                           float* __restrict__ dx) {
  __shared__ int32_t es[kMaxTopK];
  __shared__ float ds[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < kMaxTopK) {
    int32_t e = -1;
    float d = 0.0f;
    if (threadIdx.x < k) {
      e = idx[t * k + threadIdx.x];
      d = dl[t * k + threadIdx.x];
    }
    es[threadIdx.x] = (e >= 0 && e < N) ? e : -1;
    ds[threadIdx.x] = d;
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    float4 w[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k && es[j] >= 0) w[j] = *reinterpret_cast<const float4*>(w_router + (int64_t)es[j] * H + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && es[j] >= 0) {
        acc.x = fmaf(ds[j], w[j].x, acc.x);
        acc.y = fmaf(ds[j], w[j].y, acc.y);
        acc.z = fmaf(ds[j], w[j].z, acc.z);
        acc.w = fmaf(ds[j], w[j].w, acc.w);
      }
    }
    *reinterpret_cast<float4*>(dx + t * H + c) = acc;
  }
}

// 4 consecutive values at p[i..i+4) (i a multiple of 4) as floats.
template <typename T>
__device__ __forceinline__ void ld4(const T* p, int64_t i, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 raw = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    v[0] = __uint_as_float(raw.x << 16);
    v[1] = __uint_as_float(raw.x & 0xffff0000u);
    v[2] = __uint_as_float(raw.y << 16);
    v[3] = __uint_as_float(raw.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

// dW_r: one block per (expert, 1024 features), four consecutive features per thread; the
// expert's rows go in ascending order, in batches of kDwRows whose loads are all issued
// before any is added.
constexpr int kDwRows = 8;

template <typename XT>
__global__ __launch_bounds__(256) void route_bwd_dw_kernel(const float* __restrict__ dl_row,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ row_token,
                                                           const XT* __restrict__ x, int64_t T,
                                                           int H, float* __restrict__ dw) {
  const int e = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  const int lo = offsets[e], hi = offsets[e + 1];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = lo; r0 < hi; r0 += kDwRows) {
    float v[kDwRows][4], g[kDwRows];
    bool ok[kDwRows];
#pragma unroll
    for (int u = 0; u < kDwRows; ++u) {
      const int r = r0 + u;
      int64_t t = -1;
      g[u] = 0.0f;
      if (r < hi) {
        t = row_token[r];
        g[u] = dl_row[r];
      }
      ok[u] = t >= 0 && t < T;
      ld4(x, (ok[u] ? t : 0) * H + c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kDwRows; ++u)
      if (ok[u])
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(g[u], v[u][i], acc[i]);
  }
  *reinterpret_cast<float4*>(dw + (int64_t)e * H + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// ------------------------------------------------------------------------------------
// Unpermute-sum: dx_t = sum_s rows[T k + s T + t] + sum_j rows[row_of[t, j]] (+ extra_t),
// FP32 in that order, one bf16 rounding. Block (token, 1024 columns), 4 columns per thread;
// the slot rows and extra are loaded before anything is added, so a thread's loads are in
// flight together.
// ------------------------------------------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(256) void unpermute_sum_kernel(const YT* __restrict__ rows,
                                                            const int32_t* __restrict__ row_of,
                                                            const float* __restrict__ extra,
                                                            int64_t T, int H, int k, int S,
                                                            int64_t n_rows,
                                                            uint16_t* __restrict__ out) {
  __shared__ int32_t rs[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < kMaxTopK) {
    int32_t r = -1;
    if (threadIdx.x < k) r = row_of[t * k + threadIdx.x];
    rs[threadIdx.x] = (r >= 0 && r < n_rows) ? r : -1;
  }
  __syncthreads();
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float v[kMaxTopK][4], ve[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k && rs[j] >= 0) ld4(rows, (int64_t)rs[j] * H + c, v[j]);
  if (extra) ld4(extra, t * H + c, ve);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    float u[4];
    ld4(rows, (T * k + s * T + t) * H + c, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += u[i];
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k && rs[j] >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += v[j][i];
    }
  if (extra) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += ve[i];
  }
  *reinterpret_cast<uint2*>(out + t * H + c) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
}

// ------------------------------------------------------------------------------------
// Weight transposition (set-up): dst[e][c][col0 + r] = src[e][r][c] for E4M3 codes, and
// the 128x128 block scales moved with their blocks. 64x64 tiles through LDS.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_codes_kernel(const uint8_t* __restrict__ src,
                                                              int64_t R, int64_t C,
                                                              uint8_t* __restrict__ dst,
                                                              int64_t dst_cols, int64_t col0) {
  __shared__ uint8_t tile[64][65];
  const int64_t e = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint8_t* s = src + e * R * C;
  for (int i = ty; i < 64; i += 4) tile[i][tx] = s[(r0 + i) * C + c0 + tx];
  __syncthreads();
  uint8_t* d = dst + e * C * dst_cols;
  for (int i = ty; i < 64; i += 4) d[(c0 + i) * dst_cols + col0 + r0 + tx] = tile[tx][i];
}

__global__ void transpose_scales_kernel(const float* __restrict__ src, int64_t E, int64_t RB,
                                        int64_t CB, float* __restrict__ dst, int64_t dst_cb,
                                        int64_t cb0) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E * RB * CB) return;
  const int64_t e = i / (RB * CB), rb = (i / CB) % RB, cb = i % CB;
  dst[(e * CB + cb) * dst_cb + cb0 + rb] = src[i];
}

// ------------------------------------------------------------------------------------
// FFN backward helpers
// ------------------------------------------------------------------------------------

// 1x128 quantisation of one 128-wide tile per wave (2 values per lane), the forward's rule:
// s = fl32(amax / 448) (1 for a zero tile), codes = E4M3(fl32(v / s)).
__device__ __forceinline__ void quant_tile_wave(float v0, float v1, float& s, uint32_t& c0,
                                                uint32_t& c1) {
  const float amax = group_max<kWave>(fmaxf(fabsf(v0), fabsf(v1)));
  s = group_scale(amax);
  c0 = e4m3_encode(__fdiv_rn(v0, s));
  c1 = e4m3_encode(__fdiv_rn(v1, s));
}

// dy of the permuted rows, dy_r = fl32(row_gate[r] dout[row_token[r]]) (row_gate NULL: 1),
// quantised 1x128 along H: codes [rows, H] and scales chunk-major [H/128][rows]; rows
// without a token quantise as zeros. One workgroup per row; a thread takes 8 consecutive
// values of every 2048 (16 lanes per 128-wide tile), all of its loads issued before any
// tile is quantised. STEPS = ceil(H / 2048) (at most 8: H <= 16384), so a thread holds only
// the values it quantises.
template <int STEPS>
__global__ __launch_bounds__(256) void quant_dy_rows_kernel(const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ row_gate,
                                                            const int32_t* __restrict__ row_token,
                                                            int64_t n_tokens, int64_t n_rows, int C,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ s_cm) {
  const int64_t r = blockIdx.x;
  const int64_t t = row_token[r];
  const bool live = t >= 0 && t < n_tokens;
  const float gr = row_gate ? row_gate[r] : 1.0f;
  float v[STEPS][8];
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int c = u * 2048 + threadIdx.x * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
    if (live && c < C) {
      float d[8];
      ld8(dout, t * C + c, d);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = gr * d[i];
    }
  }
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int c = u * 2048 + threadIdx.x * 8;
    if (u * 2048 >= C) break;
    // amax over the tile's 16 lanes (lanes 16a .. 16a+15 hold one 128-wide tile)
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    m = fmaxf(m, __shfl_xor(m, 4, kWave));
    m = fmaxf(m, __shfl_xor(m, 8, kWave));
    if (c < C) {
      const float sc = group_scale(m);
      const uint32_t lo = e4m3_encode(__fdiv_rn(v[u][0], sc)) | (e4m3_encode(__fdiv_rn(v[u][1], sc)) << 8) |
                          (e4m3_encode(__fdiv_rn(v[u][2], sc)) << 16) | (e4m3_encode(__fdiv_rn(v[u][3], sc)) << 24);
      const uint32_t hi = e4m3_encode(__fdiv_rn(v[u][4], sc)) | (e4m3_encode(__fdiv_rn(v[u][5], sc)) << 8) |
                          (e4m3_encode(__fdiv_rn(v[u][6], sc)) << 16) | (e4m3_encode(__fdiv_rn(v[u][7], sc)) << 24);
      *reinterpret_cast<uint2*>(q + r * C + c) = make_uint2(lo, hi);
      if ((threadIdx.x & 15) == 0) s_cm[(int64_t)(c / kTile) * n_rows + r] = sc;
    }
  }
}

// SwiGLU backward on FP32 a, b, dh [rows, I]: dg = dh b silu'(a) -> dg_out, du = dh silu(a)
// -> du_out, h = silu(a) b -> dh (in place; dg_out and du_out may be a and b); and
// [dg | du] quantised 1x128 along I into codes [rows, 2I] with scales chunk-major
// [2I/128][rows]. One wave per 128-wide tile.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* a, const float* b,
                                                         float* __restrict__ dh, int64_t n_rows,
                                                         int I, float* dg_out, float* du_out,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ s_cm) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nct = I / kTile;
  if (tile >= n_rows * nct) return;
  const int64_t r = tile / nct;
  const int ct = (int)(tile % nct);
  const int64_t o = r * I + ct * kTile + 2 * lane;
  const float2 av = *reinterpret_cast<const float2*>(a + o);
  const float2 bv = *reinterpret_cast<const float2*>(b + o);
  const float2 dv = *reinterpret_cast<const float2*>(dh + o);
  float dg[2], du[2], h[2];
  const float avs[2] = {av.x, av.y}, bvs[2] = {bv.x, bv.y}, dvs[2] = {dv.x, dv.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float sg = 1.0f / (1.0f + expf(-avs[i]));
    const float si = avs[i] * sg;
    const float sd = sg * (1.0f + avs[i] * (1.0f - sg));
    dg[i] = dvs[i] * bvs[i] * sd;
    du[i] = dvs[i] * si;
    h[i] = si * bvs[i];
  }
  *reinterpret_cast<float2*>(dg_out + o) = make_float2(dg[0], dg[1]);
  *reinterpret_cast<float2*>(du_out + o) = make_float2(du[0], du[1]);
  *reinterpret_cast<float2*>(dh + o) = make_float2(h[0], h[1]);
  float s;
  uint32_t c0, c1;
  quant_tile_wave(dg[0], dg[1], s, c0, c1);
  reinterpret_cast<uint16_t*>(q + r * 2 * I + ct * kTile)[lane] = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) s_cm[(int64_t)ct * n_rows + r] = s;
  quant_tile_wave(du[0], du[1], s, c0, c1);
  reinterpret_cast<uint16_t*>(q + r * 2 * I + I + ct * kTile)[lane] = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) s_cm[(int64_t)(nct + ct) * n_rows + r] = s;
}

// Padded segment layout for the token-axis operands: expert e's rows occupy padded rows
// [poff[e], poff[e] + 128 ceil(M_e / 128)); chunk_e[g] names the expert of padded chunk g
// (-1 past the last); elong = {count, experts of more than long_ch chunks in ascending
// order}. One workgroup.
__global__ __launch_bounds__(1024) void pad_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int n_experts, int max_chunks, int long_ch,
                                                        int32_t* __restrict__ poff,
                                                        int32_t* __restrict__ chunk_e,
                                                        int32_t* __restrict__ elong) {
  __shared__ int32_t cs[1025];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int run = 0, nl = 0;
    for (int e = 0; e < n_experts; ++e) {
      cs[e] = run;
      const int m = max(offsets[e + 1] - offsets[e], 0);
      const int nch = (m + kTile - 1) / kTile;
      run += nch;
      if (nch > long_ch) elong[1 + nl++] = e;
    }
    cs[n_experts] = min(run, max_chunks);
    elong[0] = nl;
  }
  __syncthreads();
  for (int e = tid; e <= n_experts; e += 1024) poff[e] = min(cs[e], max_chunks) * kTile;
  for (int g = tid; g < max_chunks; g += 1024) chunk_e[g] = -1;
  __syncthreads();
  for (int e = tid; e < n_experts; e += 1024)
    for (int g = cs[e]; g < min(cs[e + 1], max_chunks); ++g) chunk_e[g] = e;
}

// Token-axis quantisation, transposed: for padded chunk g (128 padded rows of one expert)
// and 64 columns, column c's 128 values (rows past the segment read zero) get the scale
// s = fl32(amax / 448) and are stored as codes qt[c][128 g + i], scales s_cm[g][c].
// Source rows: src[r] (MODE 0), src[row_token[r]] (MODE 1), or src[row_token[r]] times
// row_gate[r] in one FP32 rounding (MODE 3: dy from the upstream gradient; row_gate NULL
// means 1).
// Thread (q, rg) holds columns 4q .. 4q+3 of rows 8rg .. 8rg+7: one 8- or 16-byte load per
// row (a wave's load covers four rows of 64 columns), all eight issued before any is used;
// rows without a source are not read.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void quant_tokens_kernel(const T* __restrict__ src, int64_t src_rows,
                                                           int64_t n_rows,
                                                           const int32_t* __restrict__ row_token,
                                                           const float* __restrict__ row_gate,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ poff,
                                                           const int32_t* __restrict__ chunk_e,
                                                           int C, int64_t pstride,
                                                           uint8_t* __restrict__ qt,
                                                           float* __restrict__ s_cm) {
  __shared__ float amx[4][64];
  __shared__ int64_t srow[kTile];   // source row of each of the chunk's rows, -1: zero
  __shared__ float grow[kTile];     // MODE 3: the row's gate
  __shared__ uint2 stg[64][16];     // codes of the 64 columns (128 bytes each), 8-byte
                                    // piece p of column c at p ^ ((c >> 2) & 15)
  const int64_t g = blockIdx.x;
  const int e = chunk_e[g];
  if (e < 0) return;
  const int q = threadIdx.x & 15, rg = threadIdx.x >> 4, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.y * 64 + 4 * q;           // first of this thread's four columns
  const int64_t first = offsets[e] + (g * kTile - poff[e]);   // permuted row of padded row 128 g
  const int64_t end = min((int64_t)offsets[e + 1], n_rows);
  if (threadIdx.x < kTile) {
    const int64_t r = first + threadIdx.x;
    int64_t sr = -1;
    float gv = 1.0f;
    if (r < end) {
      if (MODE == 1 || MODE == 3) {
        const int64_t t = row_token[r];
        sr = (t >= 0 && t < src_rows) ? t : -1;
        if (MODE == 3 && row_gate) gv = row_gate[r];
      } else {
        sr = r;
      }
    }
    srow[threadIdx.x] = sr;
    grow[threadIdx.x] = gv;
  }
  __syncthreads();
  const bool col_ok = c0 < C;   // C is a multiple of 128: all four columns or none
  float v[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t sr = srow[rg * 8 + i];
    v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.0f;
    if (sr >= 0 && col_ok) {
      if constexpr (sizeof(T) == 2) {
        const uint2 raw = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(src) + sr * C + c0);
        v[i][0] = __uint_as_float(raw.x << 16);
        v[i][1] = __uint_as_float(raw.x & 0xffff0000u);
        v[i][2] = __uint_as_float(raw.y << 16);
        v[i][3] = __uint_as_float(raw.y & 0xffff0000u);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + sr * C + c0);
        v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
      }
      if constexpr (MODE == 3) {
        const float gv = grow[rg * 8 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = gv * v[i][j];
      }
    }
  }
  // column maxima: this thread's 8 rows, the wave's 4 row groups (lanes 16 apart), then
  // the 4 waves through LDS
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m[j] = fmaxf(m[j], fabsf(v[i][j]));
    m[j] = fmaxf(m[j], __shfl_xor(m[j], 16, kWave));
    m[j] = fmaxf(m[j], __shfl_xor(m[j], 32, kWave));
  }
  if ((threadIdx.x & 63) < 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) amx[wave][4 * q + j] = m[j];
  }
  __syncthreads();
  float sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cc = 4 * q + j;
    sc[j] = group_scale(fmaxf(fmaxf(amx[0][cc], amx[1][cc]), fmaxf(amx[2][cc], amx[3][cc])));
  }
  // codes of column 4q + j, rows 8rg .. 8rg+7: bytes 8rg .. 8rg+7 of that column's 128
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cc = 4 * q + j;
    const uint32_t lo = e4m3_encode(__fdiv_rn(v[0][j], sc[j])) | (e4m3_encode(__fdiv_rn(v[1][j], sc[j])) << 8) |
                        (e4m3_encode(__fdiv_rn(v[2][j], sc[j])) << 16) | (e4m3_encode(__fdiv_rn(v[3][j], sc[j])) << 24);
    const uint32_t hi = e4m3_encode(__fdiv_rn(v[4][j], sc[j])) | (e4m3_encode(__fdiv_rn(v[5][j], sc[j])) << 8) |
                        (e4m3_encode(__fdiv_rn(v[6][j], sc[j])) << 16) | (e4m3_encode(__fdiv_rn(v[7][j], sc[j])) << 24);
    stg[cc][rg ^ ((cc >> 2) & 15)] = make_uint2(lo, hi);
  }
  if (rg == 0 && col_ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s_cm[g * C + c0 + j] = sc[j];
  }
  __syncthreads();
  // whole 128-byte rows of qt (8 lanes per column, 16 bytes each)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = threadIdx.x + 256 * i, cc = u >> 3, p = u & 7;
    const int col = blockIdx.y * 64 + cc;
    if (col < C) {
      const uint2 a = stg[cc][(2 * p) ^ ((cc >> 2) & 15)];
      const uint2 b = stg[cc][(2 * p + 1) ^ ((cc >> 2) & 15)];
      *reinterpret_cast<uint4*>(qt + (int64_t)col * pstride + g * kTile + p * 16) = make_uint4(a.x, a.y, b.x, b.y);
    }
  }
}

// ------------------------------------------------------------------------------------
// wgrad: out_e[n][m] = sum over expert e's padded rows p of A_T[n][p] B_T[m][p], FP8 E4M3
// operands in 128-row tiles along p with scales chunk-major (sa[g][n], sb[g][m]); each
// 128-row chunk is one MFMA per 16x16 block, promoted in FP32 by sa[n] sb[m], chunks in
// order. Output tiles are 128 x 128. The MFMA takes B_T as its first operand, so a lane's
// four results are four consecutive m of one n: one 16-byte store each (plain stores:
// measured non-temporal ones of this pattern, half cache lines per row, at 60% of the
// plain rate). Two kernels split the experts by segment length: wgrad_strip_kernel (at
// most kStripCh chunks) and wgrad_long_kernel (the rest).
// ------------------------------------------------------------------------------------
constexpr int kWgM = 128;   // output columns per tile

// Stores one lane's 4 consecutive m of one n.
template <typename OT>
__device__ __forceinline__ void wgrad_store1(OT* o, const v4f& v) {
  if constexpr (sizeof(OT) == 4) {
    *reinterpret_cast<v4f*>(o) = v;
  } else {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    const v2u pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<v2u*>(o) = pk;
  }
}

// ------------------------------------------------------------------------------------
// wgrad of short segments (at most kStripCh token chunks, as every routed expert has at a
// few thousand tokens): a workgroup keeps the expert's 128-row strip of A_T (and of A2_T),
// all of its chunks, in LDS and walks kStripMR consecutive 128-column output tiles, so per
// tile it loads only the B_T fragments and their scales. A wave's memory operations
// complete in issue order, and the loads of tile j+1 are issued before the stores of tile
// j, so the wait for them is not a wait for the stores. SHARE 1: two A strips, the same
// rows of two matrices (dW1 and dW3 share B = x); SHARE 2: two consecutive 128-row strips
// of one matrix (dW2); SHARE 0: one strip. Either way of pairing, each B load serves two
// output tiles. A wave computes all 128 rows by 32 columns of a tile.
// ------------------------------------------------------------------------------------
constexpr int kStripCh = 2;                  // chunks of a short segment
constexpr int kStripRow = kStripCh * kTile;  // LDS bytes of one strip row (16 pieces of 16)
constexpr int kStripMR = 4;                  // output tiles per workgroup (2, 3, 6, 8 and 16 measured slower)

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const v4i lds_v4i;

// s_waitcnt immediate: at most n vector-memory operations outstanding and every LDS
// operation done (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in
// bits 15:14).
constexpr int wait_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0070; }

template <typename OT, int SHARE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void wgrad_strip_kernel(
    const uint8_t* __restrict__ at, const float* __restrict__ sa, const uint8_t* __restrict__ at2,
    const float* __restrict__ sa2, const uint8_t* __restrict__ bt, const float* __restrict__ sb,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ offsets, int n_experts, int NA,
    int NB, int64_t pstride, OT* __restrict__ out, OT* __restrict__ out2) {
  static_assert(SHARE >= 0 && SHARE <= 2, "one or two A strips");
  constexpr int NS = SHARE ? 2 : 1;          // A strips, one output tile each
  constexpr int kSpanA = SHARE == 2 ? 2 * kTile : kTile;   // rows of A_T per work item
  constexpr int kStores = NS * 16;           // store instructions per wave and tile
  // strip rows of A_T: 16-byte piece s of row r holds K piece s ^ (r & 15)
  __shared__ __attribute__((aligned(16))) uint8_t lda[NS][kTile * kStripRow];
  __shared__ __attribute__((aligned(16))) float lsa[NS][kStripCh][kTile];   // A scales
  __shared__ __attribute__((aligned(16))) float lsb[2][kStripCh][kTile];    // B scales, by tile parity
  // work item: expert e (on XCD e % 8, so its B_T rows stay in one L2), kSpanA rows of A_T,
  // range of kStripMR column tiles
  const int ga = NA / kSpanA, tiles = NB / kWgM;
  const int nmr = (tiles + kStripMR - 1) / kStripMR, per_e = ga * nmr;
  const int64_t L = blockIdx.x, slot = L / 8;
  const int64_t ee = L % 8 + 8 * (slot / per_e);
  if (ee >= n_experts) return;
  const int e = (int)ee;
  const int p0 = poff[e], nch = (poff[e + 1] - p0) / kTile;
  if (nch > kStripCh) return;   // a long segment: wgrad_long_kernel
  const int it = (int)(slot % per_e);
  const int n0 = (it / nmr) * kSpanA;
  const int j0 = (it % nmr) * kStripMR, j1 = min(j0 + kStripMR, tiles);
  const int g0 = p0 / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4, lk = lg * 32;
  const int wml = wave * 32;   // the wave's 32 columns of the tile, against all 128 rows
  const int rows_e = max(offsets[e + 1] - offsets[e], 0);
  constexpr int kOut = (int)0x80000000;   // an offset past every range: reads zeros
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(at), 0, (int)((int64_t)NA * pstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(SHARE == 1 ? at2 : at), 0, (int)((int64_t)NA * pstride), 0x00020000);
  // strip w: rows n0 + sw * w of A (SHARE 2: the second strip is the next 128 rows of the
  // same matrix and output; SHARE 1: the same rows of the second matrix and output)
  constexpr int sw = SHARE == 2 ? kTile : 0;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(bt), 0, (int)((int64_t)NB * pstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sa), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(SHARE == 1 ? sa2 : sa), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sb), 0, 0x7fffffff, 0x00020000);

  // B_T fragments of one tile (this wave's 32 columns), every chunk of the segment, and the
  // tile's B scales (all 4 waves: 2 x 128 floats) into lsb[buf]
  constexpr int kSJ = 2;   // 16-column blocks per wave
  v8i B[kStripCh][kSJ];
  auto issue_b = [&](int j, int buf) __attribute__((always_inline)) {
    {
      const int v = wave * kWave + lane, ch = v >> 7, mm = v & (kTile - 1);
      const int off = ch < nch ? (int)(((int64_t)(g0 + ch) * NB + j * kWgM + mm) * 4) : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_u8*)&lsb[buf][0][0] + wave * kWave * 4, 4, off, 0, 0, 0);
    }
#pragma unroll
    for (int ch = 0; ch < kStripCh; ++ch) {
      if (ch < nch) {
        const bool live = lk < rows_e - ch * kTile;
#pragma unroll
        for (int jj = 0; jj < kSJ; ++jj) {
          const int64_t row = j * kWgM + wml + 16 * jj + lr;
          int off = live ? (int)(row * pstride + p0 + ch * kTile + lk) : kOut;
          // one load for both cases (split into two, the loads' registers would make the
          // compiler wait for every earlier store)
          asm volatile("" : "+v"(off));
          const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
          const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, off + 16, 0, 0));
          B[ch][jj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    }
  };

  // prologue: the strips and their scales (rows past the segment are stored zeros; chunks
  // past it read zeros), then the first tile's B
#pragma unroll
  for (int w = 0; w < NS; ++w) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int u = (q * 4 + wave) * kWave + lane;   // 16-byte unit of lda[w]
      const int rr = u >> 4, kp = (u & 15) ^ (rr & 15), ch = kp >> 3;
      const int off =
          ch < nch ? (int)((int64_t)(n0 + sw * w + rr) * pstride + p0 + ch * kTile + (kp & 7) * 16) : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w ? ra2 : ra, (lds_u8*)&lda[w][0] + (q * 4 + wave) * kWave * 16, 16,
                                               off, 0, 0, 0);
    }
    {
      const int v = wave * kWave + lane, ch = v >> 7, rr = v & (kTile - 1);
      const int off = ch < nch ? (int)(((int64_t)(g0 + ch) * NA + n0 + sw * w + rr) * 4) : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w ? rsa2 : rsa, (lds_u8*)&lsa[w][0][0] + wave * kWave * 4, 4, off,
                                               0, 0, 0);
    }
  }
  issue_b(j0, 0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // acc[w][i][jj]: n = n0 + 16 i + lr, m = 128 j + wml + 16 jj + 4 lg + v
  v4f acc[NS][8][kSJ];
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
#pragma unroll
    for (int w = 0; w < NS; ++w)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < kSJ; ++jj) acc[w][i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < kStripCh; ++ch) {
      if (ch < nch) {
        float4 sbm[kSJ];
#pragma unroll
        for (int jj = 0; jj < kSJ; ++jj)
          sbm[jj] = *reinterpret_cast<const float4*>(&lsb[buf][ch][wml + 16 * jj + 4 * lg]);
#pragma unroll
        for (int w = 0; w < NS; ++w) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = 16 * i + lr;   // row & 15 == lr
            const int kp = ch * 8 + lg * 2;
            const lds_u8* rp = (const lds_u8*)&lda[w][0] + row * kStripRow;
            const v4i lo = *reinterpret_cast<lds_v4i*>(rp + ((kp ^ lr) << 4));
            const v4i hi = *reinterpret_cast<lds_v4i*>(rp + (((kp + 1) ^ lr) << 4));
            const v8i A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const float san = lsa[w][ch][row];
            const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < kSJ; ++jj) {
              const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(B[ch][jj], A, z, 0, 0, 0, 127, 0, 127);
              acc[w][i][jj][0] = fmaf(d[0], san * sbm[jj].x, acc[w][i][jj][0]);
              acc[w][i][jj][1] = fmaf(d[1], san * sbm[jj].y, acc[w][i][jj][1]);
              acc[w][i][jj][2] = fmaf(d[2], san * sbm[jj].z, acc[w][i][jj][2]);
              acc[w][i][jj][3] = fmaf(d[3], san * sbm[jj].w, acc[w][i][jj][3]);
            }
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < j1) issue_b(j + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int w = 0; w < NS; ++w) {
      OT* o = (SHARE == 1 && w ? out2 : out) + ((int64_t)e * NA + sw * w) * NB;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < kSJ; ++jj)
          wgrad_store1(o + (int64_t)(n0 + 16 * i + lr) * NB + j * kWgM + wml + 16 * jj + 4 * lg, acc[w][i][jj]);
    }
    if (j + 1 < j1) {
      // the next tile's B (and every wave's scale copies) arrived; the stores stay in flight
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kStores));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  }
}

// ------------------------------------------------------------------------------------
// wgrad of long segments (more than kStripCh chunks: the shared experts, hot routed
// ones): one persistent workgroup of 8 waves per CU walks 128 x 128 output tiles of the
// experts of elist = {count, experts...} and streams each tile's token chunks through an
// LDS ring of three slots (the chunk's A_T and A2_T rows, its B_T rows and their scales,
// copied by direct buffer->LDS loads two chunks ahead, across tile boundaries). Wave w
// computes rows 64 (w >> 2) .. +64 by columns 32 (w & 3) .. +32 of the tile. A wave's
// memory operations complete in issue order; every wait counts the copies and stores
// issued after the chunk it needs, so it never waits for a finished tile's stores. Same
// products and FP32 order as wgrad_strip_kernel (SHARE 0 or 1).
// ------------------------------------------------------------------------------------
constexpr int kLongWaves = 8;
constexpr int kLongGrid = 256;   // one workgroup per CU (the ring takes 100-150 KB of LDS)

template <int NS>
struct LongSlot {
  uint8_t blk[NS + 1][kTile * kTile];   // A_T (and A2_T) rows, then B_T rows: 16-byte piece p
                                        // of row r at p ^ (r & 7)
  float sc[NS + 1][kTile];              // their scales
  float junk[kWave];                    // landing area of the waves with no scale copy
};

template <typename OT, int SHARE>
__global__ __launch_bounds__(kLongWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void wgrad_long_kernel(
    const uint8_t* __restrict__ at, const float* __restrict__ sa, const uint8_t* __restrict__ at2,
    const float* __restrict__ sa2, const uint8_t* __restrict__ bt, const float* __restrict__ sb,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ offsets, int n_experts, int NA,
    int NB, int64_t pstride, OT* __restrict__ out, OT* __restrict__ out2,
    const int32_t* __restrict__ elist) {
  static_assert(SHARE == 0 || SHARE == 1, "one or two outputs");
  constexpr int NS = SHARE == 1 ? 2 : 1;
  constexpr int kBlkCopies = kTile * kTile / (kLongWaves * kWave * 16);   // per wave per block: 2
  constexpr int kOps = (NS + 1) * kBlkCopies + 1;   // copies per wave per chunk
  constexpr int kStores = NS * 8;                   // stores per wave per tile
  static_assert(kOps + 2 * kStores <= 63, "vmcnt range");
  // three slots, used in a loop unrolled by three; each step reads one slot and fills
  // another through restrict pointers, so the compiler can see that the reads never touch
  // the copies just issued (without that it waits for them before every read)
  __shared__ __attribute__((aligned(16))) LongSlot<NS> slot0, slot1, slot2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: descriptors and LDS bases
  const int lr = lane & 15, lg = lane >> 4;
  const int wrow = (wave >> 2) * 64, wcol = (wave & 3) * 32;
  const int ga = NA / kTile, tg = NB / kWgM;
  const int ne = min(elist[0], n_experts);
  const int64_t groups = (int64_t)ga * ne;
  const int64_t items = 8 * ((groups + 7) / 8) * tg;
  constexpr int kOut = (int)0x80000000;   // an offset past every range: reads zeros
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(at), 0, (int)((int64_t)NA * pstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(SHARE == 1 ? at2 : at), 0, (int)((int64_t)NA * pstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(bt), 0, (int)((int64_t)NB * pstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sa), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(SHARE == 1 ? sa2 : sa), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sb), 0, 0x7fffffff, 0x00020000);

  // A tile of the stream: expert, first row of A_T, first row of B_T, padded-row offset
  // and chunk count (0 for the slots past the last group).
  struct Tl {
    int e, n0, m0, p0, nch;
  };
  auto tile_of = [&](int64_t L) __attribute__((always_inline)) {
    Tl t{0, 0, 0, 0, 0};
    if (L >= items) return t;
    const int64_t slot = L / 8;
    const int64_t q = (L % 8) + 8 * (slot / tg);
    if (q >= groups) return t;
    t.e = elist[1 + q / ga];
    t.n0 = (int)(q % ga) * kTile;
    t.m0 = (int)(slot % tg) * kWgM;
    t.p0 = poff[t.e];
    t.nch = (poff[t.e + 1] - t.p0) / kTile;
    return t;
  };
  // next tile of this workgroup with at least one chunk, from L on (L >= items: none)
  auto next_tile = [&](int64_t& L, Tl& t) __attribute__((always_inline)) {
    for (; L < items; L += gridDim.x) {
      t = tile_of(L);
      if (t.nch > 0) return;
    }
    t = Tl{0, 0, 0, 0, 0};
  };

  // copies of chunk c of tile t into slot S (every wave: kOps copies)
  auto issue = [&](const Tl& t, int c, LongSlot<NS>* __restrict__ Sp) __attribute__((always_inline)) {
    LongSlot<NS>& S = *Sp;
    const int64_t pc = t.p0 + (int64_t)c * kTile;
#pragma unroll
    for (int b = 0; b <= NS; ++b) {
#pragma unroll
      for (int k = 0; k < kBlkCopies; ++k) {
        const int u = (k * kLongWaves + wave) * kWave + lane;   // 16-byte unit of the block
        const int r = u >> 3, kp = (u & 7) ^ (r & 7);
        const int64_t row = (b < NS ? t.n0 : t.m0) + r;
        const int off = (int)(row * pstride + pc + kp * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b == NS ? rb : (b ? ra2 : ra),
                                                 (lds_u8*)&S.blk[b][0] + (k * kLongWaves + wave) * kWave * 16, 16,
                                                 off, 0, 0, 0);
      }
    }
    // scales: 2 (NS + 1) copies of 64 floats, by the first waves; the others copy zeros
    // into the junk area (every wave issues kOps copies)
    const int g = (int)(pc / kTile);
    const int b = wave >> 1, half = wave & 1;   // uniform
    const int idx = half * kWave + lane;
    lds_u8* const sc0 = (lds_u8*)&S.sc[0][0] + (b * kTile + half * kWave) * 4;
    if (b < NS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b == 0 ? rsa : rsa2, sc0, 4, (int)(((int64_t)g * NA + t.n0 + idx) * 4), 0,
                                               0, 0);
    else if (b == NS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, sc0, 4, (int)(((int64_t)g * NB + t.m0 + idx) * 4), 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_u8*)&S.junk[0], 4, kOut, 0, 0, 0);
  };

  // stream state: the tile and chunk being computed, and the ones being copied (two ahead)
  int64_t Lc = blockIdx.x, Ll;
  Tl tc, tl;
  next_tile(Lc, tc);
  if (tc.nch == 0) return;
  Ll = Lc;
  tl = tc;
  int cl = 0;   // chunk of tl to copy next
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (++cl == tl.nch) {
      cl = 0;
      Ll += gridDim.x;
      next_tile(Ll, tl);
    }
  };
  bool more;   // a copied chunk after the one computed next
  auto prime = [&](LongSlot<NS>* __restrict__ S0, LongSlot<NS>* __restrict__ S1) __attribute__((always_inline)) {
    issue(tl, cl, S0);
    advance_load();
    more = tl.nch > 0;
    if (more) {
      issue(tl, cl, S1);
      advance_load();
    }
  };
  prime(&slot0, &slot1);

  v4f acc[NS][4][2];
#pragma unroll
  for (int w = 0; w < NS; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[w][i][0] = acc[w][i][1] = v4f{0.f, 0.f, 0.f, 0.f};
  int cc = 0;
  int s1 = 0, s2 = 0;   // stores issued one and two steps back (per wave)
  // one chunk: compute from Sc, copy two chunks ahead into Sl; false when the stream ends
  auto step = [&](const LongSlot<NS>* __restrict__ Scp, LongSlot<NS>* __restrict__ Sl)
                  __attribute__((always_inline)) {
    const LongSlot<NS>& Sc = *Scp;
    // the copies of the next chunk (if any) and the stores of the last two steps were
    // issued after this chunk's copies
    const bool next_exists = more;
    const int after = s1 + s2;
    asm volatile("" ::: "memory");
    if (!next_exists) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    else if (after == 0) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kOps));
    else if (after == kStores) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kOps + kStores));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kOps + 2 * kStores));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // copies two chunks ahead, into the slot every wave finished with last step
    more = tl.nch > 0;
    if (more) {
      issue(tl, cl, Sl);
      advance_load();
    }
    {
      float4 sbm[2];
      v8i B[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int row = wcol + 16 * jj + lr;
        const lds_u8* rp = (const lds_u8*)&Sc.blk[NS][0] + row * kTile;
        const v4i lo = *reinterpret_cast<lds_v4i*>(rp + (((2 * lg) ^ (row & 7)) << 4));
        const v4i hi = *reinterpret_cast<lds_v4i*>(rp + (((2 * lg + 1) ^ (row & 7)) << 4));
        B[jj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        sbm[jj] = *reinterpret_cast<const float4*>(&Sc.sc[NS][wcol + 16 * jj + 4 * lg]);
      }
#pragma unroll
      for (int w = 0; w < NS; ++w) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wrow + 16 * i + lr;
          const lds_u8* rp = (const lds_u8*)&Sc.blk[w][0] + row * kTile;
          const v4i lo = *reinterpret_cast<lds_v4i*>(rp + (((2 * lg) ^ (row & 7)) << 4));
          const v4i hi = *reinterpret_cast<lds_v4i*>(rp + (((2 * lg + 1) ^ (row & 7)) << 4));
          const v8i A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const float san = Sc.sc[w][row];
          const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(B[jj], A, z, 0, 0, 0, 127, 0, 127);
            acc[w][i][jj][0] = fmaf(d[0], san * sbm[jj].x, acc[w][i][jj][0]);
            acc[w][i][jj][1] = fmaf(d[1], san * sbm[jj].y, acc[w][i][jj][1]);
            acc[w][i][jj][2] = fmaf(d[2], san * sbm[jj].z, acc[w][i][jj][2]);
            acc[w][i][jj][3] = fmaf(d[3], san * sbm[jj].w, acc[w][i][jj][3]);
          }
        }
      }
    }
    s2 = s1;
    s1 = 0;
    if (++cc == tc.nch) {
      // the tile is done: store it, start the next one
#pragma unroll
      for (int w = 0; w < NS; ++w) {
        OT* o = (w ? out2 : out) + (int64_t)tc.e * NA * NB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            wgrad_store1(o + (int64_t)(tc.n0 + wrow + 16 * i + lr) * NB + tc.m0 + wcol + 16 * jj + 4 * lg,
                         acc[w][i][jj]);
            acc[w][i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
          }
      }
      s1 = kStores;
      if (!next_exists) return false;
      cc = 0;
      Lc += gridDim.x;
      next_tile(Lc, tc);
    }
    return true;
  };
  // the first three steps are peeled: entering the loop from the prologue, the compiler's
  // wait analysis cannot tell the slots apart and waits for every copy in flight
  if (step(&slot0, &slot2) && step(&slot1, &slot0) && step(&slot2, &slot1))
    while (step(&slot0, &slot2) && step(&slot1, &slot0) && step(&slot2, &slot1)) {
    }
}

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of the FFN backward.
struct BwdLayout {
  size_t plan, dyq, dys, xgs, fa, fb, fdh, q3, s3, poff, chunk_e, elong, dyt, dyts, xt, xts, ht,
      hts, gt, gts, ut, uts, total;
  int64_t max_chunks, pstride;
};

inline BwdLayout bwd_layout(const moe_config* c, int32_t E, int64_t n_rows) {
  BwdLayout L;
  const int64_t H = c->hidden, I = c->inter;
  L.max_chunks = (n_rows + kTile - 1) / kTile + E;
  L.pstride = L.max_chunks * kTile;
  const int64_t P = L.pstride, G = L.max_chunks;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  L.plan = take(ffn_plan_bytes(E, n_rows));
  L.dyq = take((size_t)n_rows * H);
  L.dys = take((size_t)n_rows * (H / kTile) * 4);
  L.xgs = take((size_t)n_rows * (H / kTile) * 4);
  L.fa = take((size_t)n_rows * I * 4);
  L.fb = take((size_t)n_rows * I * 4);
  L.fdh = take((size_t)n_rows * I * 4);
  L.q3 = take((size_t)n_rows * 2 * I);
  L.s3 = take((size_t)n_rows * (2 * I / kTile) * 4);
  L.poff = take((size_t)(E + 1) * 4);
  L.chunk_e = take((size_t)G * 4);
  L.elong = take((size_t)(E + 1) * 4);
  L.dyt = take((size_t)H * P);
  L.dyts = take((size_t)G * H * 4);
  L.xt = take((size_t)H * P);
  L.xts = take((size_t)G * H * 4);
  L.ht = take((size_t)I * P);
  L.hts = take((size_t)G * I * 4);
  L.gt = take((size_t)I * P);
  L.gts = take((size_t)G * I * 4);
  L.ut = take((size_t)I * P);
  L.uts = take((size_t)G * I * 4);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace moe

using namespace moe;

// ------------------------------------------------------------------------------------
// Entry points
// ------------------------------------------------------------------------------------
extern "C" moe_status moe_combine_backward(const moe_config* cfg, int64_t T, const uint16_t* dout,
                                           const void* y_rows, moe_dtype yt, const int32_t* row_of,
                                           const float* topk_gate, float* row_gate, float* dgate,
                                           void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > 0x7fffffff) return MOE_ERR_SHAPE;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!dout || !y_rows || !row_of || !topk_gate || !row_gate || !dgate) return MOE_ERR_NULL;
  const int64_t n_rows = T * (cfg->top_k + cfg->n_shared);
  hipStream_t s = as_stream(stream);
  if (yt == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd_kernel<uint16_t>, dim3((unsigned)T), dim3(256), 0, s, dout,
                       static_cast<const uint16_t*>(y_rows), row_of, topk_gate, T, cfg->hidden,
                       cfg->top_k, cfg->n_shared, n_rows, row_gate, dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3((unsigned)T), dim3(256), 0, s, dout,
                       static_cast<const float*>(y_rows), row_of, topk_gate, T, cfg->hidden,
                       cfg->top_k, cfg->n_shared, n_rows, row_gate, dgate);
  return launch_status();
}

extern "C" size_t moe_route_backward_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_config(cfg) != MOE_OK || T <= 0) return 0;
  return al256((size_t)T * cfg->top_k * 4) + al256((size_t)T * cfg->top_k * 4);
}

extern "C" moe_status moe_route_backward(const moe_config* cfg, int64_t T, const void* x,
                                         moe_dtype xt, const float* w_router, const float* scores,
                                         const int32_t* topk_idx, const float* dgate,
                                         const int32_t* offsets, const int32_t* row_token,
                                         const int32_t* row_of, float* dx, float* dw_router,
                                         void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > 0x7fffffff) return MOE_ERR_SHAPE;
  if (xt != MOE_BF16 && xt != MOE_F32) return MOE_ERR_DTYPE;
  if (!dw_router || !offsets) return MOE_ERR_NULL;
  const int N = cfg->n_routed, k = cfg->top_k, H = cfg->hidden;
  if (T > 0 && (!x || !w_router || !scores || !topk_idx || !dgate || !row_token || !row_of || !dx))
    return MOE_ERR_NULL;
  const size_t need = moe_route_backward_workspace_bytes(cfg, T);
  if (T > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int64_t pairs = T * k;
  float* dl = static_cast<float*>(ws);
  float* dl_row = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + al256((size_t)pairs * 4));
  if (T > 0) {
    hipLaunchKernelGGL(route_bwd_gates_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                       scores, topk_idx, dgate, row_of, T, N, k, cfg->routed_scaling, pairs, dl,
                       dl_row);
    hipLaunchKernelGGL(route_bwd_dx_kernel, dim3((unsigned)T), dim3(256), 0, s, dl, topk_idx,
                       w_router, N, k, H, dx);
  }
  const dim3 g((unsigned)((H / 4 + 255) / 256), (unsigned)N);
  if (xt == MOE_BF16)
    hipLaunchKernelGGL(route_bwd_dw_kernel<uint16_t>, g, dim3(256), 0, s, dl_row, offsets, row_token,
                       static_cast<const uint16_t*>(x), T, H, dw_router);
  else
    hipLaunchKernelGGL(route_bwd_dw_kernel<float>, g, dim3(256), 0, s, dl_row, offsets, row_token,
                       static_cast<const float*>(x), T, H, dw_router);
  return launch_status();
}

extern "C" moe_status moe_unpermute_sum(const moe_config* cfg, int64_t T, const void* rows,
                                        moe_dtype rt, const int32_t* row_of, const float* extra,
                                        uint16_t* out, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > 0x7fffffff) return MOE_ERR_SHAPE;
  if (rt != MOE_BF16 && rt != MOE_F32) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!rows || !row_of || !out) return MOE_ERR_NULL;
  const int64_t n_rows = T * (cfg->top_k + cfg->n_shared);
  hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)T, (unsigned)((cfg->hidden + 1023) / 1024));
  if (rt == MOE_BF16)
    hipLaunchKernelGGL(unpermute_sum_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(rows), row_of, extra, T, cfg->hidden, cfg->top_k,
                       cfg->n_shared, n_rows, out);
  else
    hipLaunchKernelGGL(unpermute_sum_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(rows), row_of, extra, T, cfg->hidden, cfg->top_k,
                       cfg->n_shared, n_rows, out);
  return launch_status();
}

extern "C" moe_status moe_transpose_fp8_blocks(int64_t E, int64_t R, int64_t C, const uint8_t* src,
                                               const float* src_scales, uint8_t* dst,
                                               float* dst_scales, int64_t dst_cols, int64_t col0,
                                               void* stream) {
  if (E < 0 || R < 0 || C < 0 || R % kTile || C % kTile || dst_cols % kTile || col0 % kTile ||
      col0 < 0 || col0 + R > dst_cols || E > 65535 || R / 64 > 65535)
    return MOE_ERR_SHAPE;
  if (E == 0 || R == 0 || C == 0) return MOE_OK;
  if (!src || !src_scales || !dst || !dst_scales) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(transpose_codes_kernel, dim3((unsigned)(C / 64), (unsigned)(R / 64), (unsigned)E),
                     dim3(256), 0, s, src, R, C, dst, dst_cols, col0);
  const int64_t n = E * (R / kTile) * (C / kTile);
  hipLaunchKernelGGL(transpose_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     src_scales, E, R / kTile, C / kTile, dst_scales, dst_cols / kTile, col0 / kTile);
  return launch_status();
}

extern "C" size_t moe_grouped_ffn_backward_workspace_bytes(const moe_config* cfg, int32_t n_experts,
                                                           int64_t n_rows) {
  if (check_config(cfg) != MOE_OK || n_experts < 1 || n_rows < 0) return 0;
  return bwd_layout(cfg, n_experts, n_rows).total;
}

extern "C" moe_status moe_grouped_ffn_fp8_backward(
    const moe_config* cfg, int32_t n_experts, int64_t n_rows, int64_t n_tokens, const uint8_t* xq,
    const float* xs, const void* x, moe_dtype xt, const int32_t* row_token, const int32_t* offsets,
    const uint8_t* w1, const float* w1s, const uint8_t* w3, const float* w3s, const uint8_t* w2t,
    const float* w2ts, const uint8_t* w13t, const float* w13ts, const float* a_saved,
    const float* b_saved, const uint16_t* dout, const float* row_gate, void* dx_rows,
    moe_dtype dxt, void* dw1, void* dw3, void* dw2, moe_dtype dwt, void* ws, size_t ws_bytes,
    void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->scale_mode != 0) return MOE_ERR_UNSUPPORTED;
  if (n_experts < 1 || n_experts > 1024 || n_rows < 0 || n_rows >= ((int64_t)1 << 31) ||
      n_tokens < 0 || n_tokens >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (xt != MOE_BF16 && xt != MOE_F32) return MOE_ERR_DTYPE;
  if (dxt != MOE_BF16 && dxt != MOE_F32) return MOE_ERR_DTYPE;
  if (dwt != MOE_BF16 && dwt != MOE_F32) return MOE_ERR_DTYPE;
  const int64_t H = cfg->hidden, I = cfg->inter;
  const BwdLayout L = bwd_layout(cfg, n_experts, n_rows);
  // 32-bit offsets inside the grouped GEMM and the transposed operands
  if (n_rows * H >= ((int64_t)1 << 32) || n_rows * 2 * I >= ((int64_t)1 << 32) ||
      n_rows * (H / kTile) * 4 >= ((int64_t)1 << 31) || L.max_chunks >= ((int64_t)1 << 24) ||
      H > 16384 || 2 * I > 16384 || std::max(H, I) * L.pstride >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!offsets || !dw1 || !dw3 || !dw2) return MOE_ERR_NULL;
  if (n_rows > 0 && (!row_token || !w1 || !w1s || !w3 || !w3s || !w2t || !w2ts || !w13t || !w13ts ||
                     !dx_rows))
    return MOE_ERR_NULL;
  // with the forward's SwiGLU inputs at hand, only h is recomputed (from them)
  const bool saved = a_saved != nullptr || b_saved != nullptr;
  if (saved && (!a_saved || !b_saved)) return MOE_ERR_NULL;
  if (n_tokens > 0 && (!x || !dout || (!saved && (!xq || !xs)))) return MOE_ERR_NULL;
  // the token-axis quantisers read x and dout rows in 8- and 16-byte pieces
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dout)) & 15) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  void* plan = base + L.plan;
  uint8_t* dyq = base + L.dyq;
  float* dys = reinterpret_cast<float*>(base + L.dys);
  float* xgs = reinterpret_cast<float*>(base + L.xgs);
  float* fa = reinterpret_cast<float*>(base + L.fa);
  float* fb = reinterpret_cast<float*>(base + L.fb);
  float* fdh = reinterpret_cast<float*>(base + L.fdh);
  uint8_t* q3 = base + L.q3;
  float* s3 = reinterpret_cast<float*>(base + L.s3);
  int32_t* poff = reinterpret_cast<int32_t*>(base + L.poff);
  int32_t* chunk_e = reinterpret_cast<int32_t*>(base + L.chunk_e);
  int32_t* elong = reinterpret_cast<int32_t*>(base + L.elong);
  const int64_t P = L.pstride, G = L.max_chunks;
  moe_status r;
  hipLaunchKernelGGL(pad_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, n_experts, (int)G, kStripCh, poff,
                     chunk_e, elong);
  if (n_rows > 0) {
    r = ffn_plan_launch(offsets, n_experts, n_rows, plan, s);
    if (r != MOE_OK) return r;
    // dgrad of the down projection and the recomputed gate/up inputs (K = H)
    const int64_t it = n_rows * (I / kTile);
    const dim3 gq((unsigned)n_rows);
    switch ((H + 2047) / 2048) {
#define MOE_QDY(n)                                                                                  \
  case n:                                                                                          \
    hipLaunchKernelGGL(quant_dy_rows_kernel<n>, gq, dim3(256), 0, s, dout, row_gate, row_token, \
                       n_tokens, n_rows, (int)H, dyq, dys);                                        \
    break;
      MOE_QDY(1) MOE_QDY(2) MOE_QDY(3) MOE_QDY(4) MOE_QDY(5) MOE_QDY(6) MOE_QDY(7) MOE_QDY(8)
#undef MOE_QDY
      default: return MOE_ERR_UNSUPPORTED;
    }
    if (!saved && (r = ffn_recompute_launch(plan, n_experts, n_rows, n_tokens, xq, xs, row_token, w1,
                                            w1s, w3, w3s, (int)H, (int)I, xgs, fa, fb, s)) != MOE_OK)
      return r;
    if ((r = ffn_grouped_gemm_launch(plan, n_experts, n_rows, dyq, dys, w2t, w2ts, (int)I, (int)H, fdh,
                                     MOE_F32, s)) != MOE_OK)
      return r;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((it + 3) / 4)), dim3(256), 0, s,
                       saved ? a_saved : fa, saved ? b_saved : fb, fdh, n_rows, (int)I, fa, fb, q3, s3);
    // dgrad of gate/up (K = 2I)
    if ((r = ffn_grouped_gemm_launch(plan, n_experts, n_rows, q3, s3, w13t, w13ts, (int)H, (int)(2 * I),
                                     dx_rows, dxt, s)) != MOE_OK)
      return r;
  }
  // token-axis operands of the wgrad GEMMs
  uint8_t* dyt = base + L.dyt;
  float* dyts = reinterpret_cast<float*>(base + L.dyts);
  uint8_t* xtt = base + L.xt;
  float* xts = reinterpret_cast<float*>(base + L.xts);
  uint8_t* htt = base + L.ht;
  float* hts = reinterpret_cast<float*>(base + L.hts);
  uint8_t* gtt = base + L.gt;
  float* gts = reinterpret_cast<float*>(base + L.gts);
  uint8_t* utt = base + L.ut;
  float* uts = reinterpret_cast<float*>(base + L.uts);
  if (n_rows > 0) {
    const dim3 gh((unsigned)G, (unsigned)((H + 63) / 64)), gi((unsigned)G, (unsigned)((I + 63) / 64));
    hipLaunchKernelGGL((quant_tokens_kernel<uint16_t, 3>), gh, dim3(256), 0, s, dout, n_tokens, n_rows,
                       row_token, row_gate, offsets, poff, chunk_e, (int)H, P, dyt, dyts);
    if (xt == MOE_BF16)
      hipLaunchKernelGGL((quant_tokens_kernel<uint16_t, 1>), gh, dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), n_tokens, n_rows, row_token, nullptr, offsets, poff,
                         chunk_e, (int)H, P, xtt, xts);
    else
      hipLaunchKernelGGL((quant_tokens_kernel<float, 1>), gh, dim3(256), 0, s,
                         static_cast<const float*>(x), n_tokens, n_rows, row_token, nullptr, offsets, poff,
                         chunk_e, (int)H, P, xtt, xts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fdh, n_rows, n_rows, row_token,
                       nullptr, offsets, poff, chunk_e, (int)I, P, htt, hts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fa, n_rows, n_rows, row_token,
                       nullptr, offsets, poff, chunk_e, (int)I, P, gtt, gts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fb, n_rows, n_rows, row_token,
                       nullptr, offsets, poff, chunk_e, (int)I, P, utt, uts);
  }
  // wgrad GEMMs (every expert's gradient written; zero for an expert without rows): short
  // segments (at most kStripCh chunks, every expert without rows included) by strips, the
  // others (listed in elong) by the persistent long-segment kernel, one workgroup per CU
  // strip grid: 8 XCDs x ceil(E / 8) experts x strips x ranges of kStripMR tiles
  auto sgrid = [&](int64_t NA, int64_t NB, int64_t span) {
    const int64_t nmr = (NB / kWgM + kStripMR - 1) / kStripMR;
    return dim3((unsigned)(8 * (((int64_t)n_experts + 7) / 8) * (NA / span) * nmr));
  };
  auto run = [&](auto* o1, auto* o3, auto* o2) {
    using OT = std::remove_pointer_t<decltype(o1)>;
    // dW2 = dy^T h: two 128-row strips of dy_T per work item where H allows (each B load
    // then serves two output tiles, as for dW1 and dW3 below)
    if (H % (2 * kTile) == 0)
      hipLaunchKernelGGL((wgrad_strip_kernel<OT, 2>), sgrid(H, I, 2 * kTile), dim3(256), 0, s, dyt, dyts, nullptr,
                         nullptr, htt, hts, poff, offsets, n_experts, (int)H, (int)I, P, o2, nullptr);
    else
      hipLaunchKernelGGL((wgrad_strip_kernel<OT, 0>), sgrid(H, I, kTile), dim3(256), 0, s, dyt, dyts, nullptr,
                         nullptr, htt, hts, poff, offsets, n_experts, (int)H, (int)I, P, o2, nullptr);
    hipLaunchKernelGGL((wgrad_long_kernel<OT, 0>), dim3(kLongGrid), dim3(kLongWaves * kWave), 0, s, dyt, dyts,
                       nullptr, nullptr, htt, hts, poff, offsets, n_experts, (int)H, (int)I, P, o2, nullptr, elong);
    // dW1 = dg^T x and dW3 = du^T x, sharing x
    hipLaunchKernelGGL((wgrad_strip_kernel<OT, 1>), sgrid(I, H, kTile), dim3(256), 0, s, gtt, gts, utt, uts, xtt, xts,
                       poff, offsets, n_experts, (int)I, (int)H, P, o1, o3);
    hipLaunchKernelGGL((wgrad_long_kernel<OT, 1>), dim3(kLongGrid), dim3(kLongWaves * kWave), 0, s, gtt, gts, utt,
                       uts, xtt, xts, poff, offsets, n_experts, (int)I, (int)H, P, o1, o3, elong);
  };
  if (dwt == MOE_F32)
    run(static_cast<float*>(dw1), static_cast<float*>(dw3), static_cast<float*>(dw2));
  else
    run(static_cast<uint16_t*>(dw1), static_cast<uint16_t*>(dw3), static_cast<uint16_t*>(dw2));
  return launch_status();
}
