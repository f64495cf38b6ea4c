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
//   combine backward   dy rows (gate x dout, FP32) and the gates' gradient (dot products);
//   router backward    gate gradient -> affinity -> logit gradient (FP32), then dx of the
//                      router GEMM and dW_r summed per expert in segment order;
//   FFN backward       per expert segment, on the forward's tile plan:
//     dy  -> 1x128 along H                  (dgrad operand)
//     a = xq W1^T, b = xq W3^T              (the forward's gate/up launch, FP32 out)
//     dh = dy W2                            (FP8 grouped GEMM, K = H, FP32 out)
//     dg, du, h (FP32) -> [dg | du] 1x128 along I   (dgrad operand, K = 2I)
//     dx_rows = [dg | du] [W1 ; W3]         (one FP8 grouped GEMM on [W1^T | W3^T])
//     dy, h, dg, du, x  -> 128-row tiles along the token axis, stored transposed
//     dW2 = dy^T h; dW1 = dg^T x and dW3 = du^T x in one launch   (FP8 wgrad, K = tokens)
//   unpermute-sum      dx_t = sum of its rows' dx (+ the router's dx), FP32, bf16 out.
#include "common.h"
#include "ffn_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float ld_val(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  else
    return reinterpret_cast<const float*>(p)[i];
}

template <typename T>
__device__ __forceinline__ void st_val(T* p, int64_t i, float v) {
  if constexpr (sizeof(T) == 2)
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    reinterpret_cast<float*>(p)[i] = v;
}

// 8 consecutive values at p[i..i+8) (i a multiple of 8) as floats / stored from floats.
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

__device__ __forceinline__ void st8(float* p, int64_t i, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
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
// Combine backward: one block per token.
// ------------------------------------------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dout,
                                                          const YT* __restrict__ y_rows,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ gate,
                                                          int64_t T, int H, int k, int S,
                                                          int64_t n_rows, float* __restrict__ dy,
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
    rows[threadIdx.x] = (r >= 0 && r < n_rows) ? r : -1;
    g[threadIdx.x] = gv;
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
    for (int s = 0; s < S; ++s) st8(dy, (T * k + s * T + t) * H + c, d);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && rows[j] >= 0) {
        const int64_t o = (int64_t)rows[j] * H + c;
        float y[8], v[8];
        ld8(y_rows, o, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = g[j] * d[i];
          part[j] = fmaf(d[i], y[i], part[j]);
        }
        st8(dy, o, v);
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

template <typename XT>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(const float* __restrict__ dl,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ w_router,
                                                           int N, int k, int H,
                                                           float* __restrict__ dx) {
  __shared__ int32_t es[kMaxTopK];
  __shared__ float ds[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    const int e = idx[t * k + threadIdx.x];
    es[threadIdx.x] = (e >= 0 && e < N) ? e : -1;
    ds[threadIdx.x] = dl[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j)
      if (es[j] >= 0) acc = fmaf(ds[j], w_router[(int64_t)es[j] * H + c], acc);
    dx[t * H + c] = acc;
  }
}

template <typename XT>
__global__ __launch_bounds__(256) void route_bwd_dw_kernel(const float* __restrict__ dl_row,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ row_token,
                                                           const XT* __restrict__ x, int64_t T,
                                                           int H, float* __restrict__ dw) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H) return;
  const int lo = offsets[e], hi = offsets[e + 1];
  float acc = 0.0f;
  for (int r = lo; r < hi; ++r) {
    const int32_t t = row_token[r];
    if (t >= 0 && t < T) acc = fmaf(dl_row[r], ld_val(x, (int64_t)t * H + c), acc);
  }
  dw[(int64_t)e * H + c] = acc;
}

// ------------------------------------------------------------------------------------
// Unpermute-sum: dx_t = sum_s rows[T k + s T + t] + sum_j rows[row_of[t, j]] (+ extra_t),
// FP32 in that order, one bf16 rounding.
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
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    for (int s = 0; s < S; ++s) {
      ld8(rows, (T * k + s * T + t) * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    for (int j = 0; j < k; ++j) {
      if (rs[j] >= 0) {
        ld8(rows, (int64_t)rs[j] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    if (extra) {
      ld8(extra, t * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
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

// dy [rows, H] FP32 -> codes [rows, H] and scales chunk-major [H/128][rows]; rows without
// a token (row_token < 0) quantise as zeros. One workgroup per row; each wave takes every
// fourth 128-wide tile, kQB tiles' loads in flight before any is quantised.
constexpr int kQB = 8;

__global__ __launch_bounds__(256) void quant_rows_kernel(const float* __restrict__ v,
                                                         const int32_t* __restrict__ row_token,
                                                         int64_t n_rows, int C,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ s_cm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = blockIdx.x;
  const int nct = C / kTile;
  const bool live = row_token == nullptr || row_token[r] >= 0;
  for (int t0 = wave; t0 < nct; t0 += 4 * kQB) {
    float2 x[kQB];
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const int ct = min(t0 + 4 * u, nct - 1);
      x[u] = *reinterpret_cast<const float2*>(v + r * C + ct * kTile + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const int ct = t0 + 4 * u;
      if (ct < nct) {
        float s;
        uint32_t c0, c1;
        quant_tile_wave(live ? x[u].x : 0.0f, live ? x[u].y : 0.0f, s, c0, c1);
        reinterpret_cast<uint16_t*>(q + r * C + ct * kTile)[lane] = (uint16_t)(c0 | (c1 << 8));
        if (lane == 0) s_cm[(int64_t)ct * n_rows + r] = s;
      }
    }
  }
}

// SwiGLU backward on FP32 a, b, dh [rows, I], in place: a <- dg = dh b silu'(a),
// b <- du = dh silu(a), dh <- h = silu(a) b; and [dg | du] quantised 1x128 along I into
// codes [rows, 2I] with scales chunk-major [2I/128][rows]. One wave per 128-wide tile.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(float* __restrict__ a, float* __restrict__ b,
                                                         float* __restrict__ dh, int64_t n_rows,
                                                         int I, uint8_t* __restrict__ q,
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
  *reinterpret_cast<float2*>(a + o) = make_float2(dg[0], dg[1]);
  *reinterpret_cast<float2*>(b + o) = make_float2(du[0], du[1]);
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
// (-1 past the last). One workgroup.
__global__ __launch_bounds__(1024) void pad_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int n_experts, int max_chunks,
                                                        int32_t* __restrict__ poff,
                                                        int32_t* __restrict__ chunk_e) {
  __shared__ int32_t cs[1025];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < n_experts; ++e) {
      cs[e] = run;
      const int m = max(offsets[e + 1] - offsets[e], 0);
      run += (m + kTile - 1) / kTile;
    }
    cs[n_experts] = min(run, max_chunks);
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
// Source rows: src[r] (MODE 0), src[row_token[r]] (MODE 1), or src[r] only where
// row_token[r] >= 0 (MODE 2).
template <typename T, int MODE>
__global__ __launch_bounds__(256) void quant_tokens_kernel(const T* __restrict__ src, int64_t src_rows,
                                                           int64_t n_rows,
                                                           const int32_t* __restrict__ row_token,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ poff,
                                                           const int32_t* __restrict__ chunk_e,
                                                           int C, int64_t pstride,
                                                           uint8_t* __restrict__ qt,
                                                           float* __restrict__ s_cm) {
  __shared__ float amx[4][64];
  __shared__ int64_t srow[kTile];   // source row of each of the chunk's rows, -1: zero
  __shared__ uint4 stg[64][8];      // codes of the 64 columns (128 bytes each), 16-byte
                                    // segment q of column c at q ^ (c & 7)
  const int64_t g = blockIdx.x;
  const int e = chunk_e[g];
  if (e < 0) return;
  const int cg = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int c = blockIdx.y * 64 + cg;
  const int64_t first = offsets[e] + (g * kTile - poff[e]);   // permuted row of padded row 128 g
  const int64_t end = min((int64_t)offsets[e + 1], n_rows);
  if (threadIdx.x < kTile) {
    const int64_t r = first + threadIdx.x;
    int64_t sr = -1;
    if (r < end) {
      if (MODE == 1) {
        const int64_t t = row_token[r];
        sr = (t >= 0 && t < src_rows) ? t : -1;
      } else if (MODE == 2) {
        sr = row_token[r] >= 0 ? r : -1;
      } else {
        sr = r;
      }
    }
    srow[threadIdx.x] = sr;
  }
  __syncthreads();
  // all 32 loads of a thread are issued before any is used (rows without a source read
  // row 0 and are dropped)
  const int cc = min(c, C - 1);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t sr = srow[rg * 32 + i];
    v[i] = ld_val(src, (sr >= 0 ? sr : 0) * C + cc);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = srow[rg * 32 + i] >= 0 ? v[i] : 0.0f;
    m = fmaxf(m, fabsf(v[i]));
  }
  amx[rg][cg] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(amx[0][cg], amx[1][cg]), fmaxf(amx[2][cg], amx[3][cg]));
  const float s = group_scale(amax);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = e4m3_encode(__fdiv_rn(v[4 * i], s)) | (e4m3_encode(__fdiv_rn(v[4 * i + 1], s)) << 8) |
           (e4m3_encode(__fdiv_rn(v[4 * i + 2], s)) << 16) | (e4m3_encode(__fdiv_rn(v[4 * i + 3], s)) << 24);
  // through LDS, so that every store writes whole 128-byte rows of qt (8 lanes per row)
  stg[cg][(2 * rg) ^ (cg & 7)] = make_uint4(w[0], w[1], w[2], w[3]);
  stg[cg][(2 * rg + 1) ^ (cg & 7)] = make_uint4(w[4], w[5], w[6], w[7]);
  if (rg == 0 && c < C) s_cm[g * C + c] = s;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = threadIdx.x + 256 * i, cc = u >> 3, q = u & 7;
    const int col = blockIdx.y * 64 + cc;
    if (col < C)
      *reinterpret_cast<uint4*>(qt + (int64_t)col * pstride + g * kTile + q * 16) = stg[cc][q ^ (cc & 7)];
  }
}

// ------------------------------------------------------------------------------------
// wgrad: out_e[n][m] = sum over expert e's padded rows p of A_T[n][p] B_T[m][p], FP8 E4M3
// operands in 128-row tiles along p with scales chunk-major (sa[g][n], sb[g][m]); each
// 128-row chunk is one MFMA per 16x16 block, promoted in FP32 by sa[n] sb[m]. A 256-thread
// workgroup computes a 128 x kWgM output tile, each wave 64 x kWgM/2 (4 x kWJ blocks; at
// 128 x 64 with four waves per SIMD it measured 7% slower: twice the A loads). The
// MFMA takes B_T as its first operand, so a lane's four results are four consecutive m of
// one n: one 16-byte store each (plain stores: measured non-temporal ones of this pattern,
// half cache lines per row, at 60% of the plain rate).
// ------------------------------------------------------------------------------------
constexpr int kWJ = 4;              // 16-column blocks per wave
constexpr int kWgM = 32 * kWJ;      // output columns per workgroup

// Stores one wave's 64 x 64 result: lane values are 4 consecutive m of one n.
template <typename OT>
__device__ __forceinline__ void wgrad_store(OT* o, int NB, int wn, int wm, int lr, int lg,
                                            const v4f (&acc)[4][kWJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < kWJ; ++j) {
      const int64_t off = (int64_t)(wn + 16 * i + lr) * NB + wm + 16 * j + 4 * lg;
      if constexpr (sizeof(OT) == 4) {
        *reinterpret_cast<v4f*>(o + off) = acc[i][j];
      } else {
        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
        const v2u pk = {pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
        *reinterpret_cast<v2u*>(o + off) = pk;
      }
    }
  }
}

// SHARE 1: two gradients that share B_T (dW1 = dg^T x and dW3 = du^T x) in one launch: each
// workgroup loads the B fragments once and runs both A operands against them (measured
// 7.8 ms for the pair at the V3 shape against 2 x 5.0 ms for two launches).
// SHARE 2: one gradient, two adjacent 128-column tiles per workgroup sharing the A
// fragments (out2 unused; the second tile's columns start 128 after the first's).
template <typename OT, int SHARE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void wgrad_kernel(
    const uint8_t* __restrict__ at, const float* __restrict__ sa, const uint8_t* __restrict__ at2,
    const float* __restrict__ sa2, const uint8_t* __restrict__ bt, const float* __restrict__ sb,
    const int32_t* __restrict__ poff, int n_experts, int NA, int NB, int64_t pstride,
    OT* __restrict__ out, OT* __restrict__ out2) {
  // A group is the NB/128 tiles that share one 128-row block of A_T. Group q runs on XCD
  // q % 8, its tiles on consecutive slots there (the A rows stay in that L2), and each
  // expert's groups spread over all XCDs, so a long segment (a shared expert) is split
  // evenly instead of loading one XCD.
  constexpr int kSpan = SHARE == 2 ? 2 * kWgM : kWgM;   // output columns per workgroup
  const int ga = NA / kTile, tg = NB / kSpan;
  const int64_t groups = (int64_t)ga * n_experts;
  const int64_t L = blockIdx.x;
  const int64_t slot = L / 8;
  const int64_t q = (L % 8) + 8 * (slot / tg);
  if (q >= groups) return;
  const int e = (int)(q / ga);
  const int n0 = (int)(q % ga) * kTile, m0 = (int)(slot % tg) * kSpan;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = n0 + (wave >> 1) * 64, wm = m0 + (wave & 1) * (kWgM / 2);
  const int p0 = poff[e], nch = (poff[e + 1] - p0) / kTile;
  const int lr = lane & 15, lg = lane >> 4, lk = lg * 32;

  // acc[i][j]: n = wn + 16 i + lr, m = wm + 16 j + 4 lg + v; acc2: the second gradient
  // (SHARE 1) or the columns 128 further on (SHARE 2)
  v4f acc[4][kWJ], acc2[4][kWJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWJ; ++j) acc[i][j] = acc2[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](const uint8_t* aa, const float* ss, int64_t p, int64_t g, v8i (&A)[4],
                    float (&san)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4* pa = reinterpret_cast<const uint4*>(aa + (int64_t)(wn + 16 * i + lr) * pstride + p + lk);
      const uint4 a0 = pa[0], a1 = pa[1];
      A[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      san[i] = ss[g * NA + wn + 16 * i + lr];
    }
  };
  auto load_b = [&](int mb, int64_t p, int64_t g, v8i (&B)[kWJ], float4 (&sbm)[kWJ])
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kWJ; ++j) {
      const uint4* pb = reinterpret_cast<const uint4*>(bt + (int64_t)(mb + 16 * j + lr) * pstride + p + lk);
      const uint4 b0 = pb[0], b1 = pb[1];
      B[j] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    }
#pragma unroll
    for (int j = 0; j < kWJ; ++j) sbm[j] = *reinterpret_cast<const float4*>(sb + g * NB + mb + 16 * j + 4 * lg);
  };
  auto mma = [&](const v8i (&A)[4], const float (&san)[4], const v8i (&B)[kWJ],
                 const float4 (&sbm)[kWJ], v4f (&ac)[4][kWJ]) __attribute__((always_inline)) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < kWJ; ++j) {
        // rows of the result: m (from B_T), columns: n (from A_T)
        const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(B[j], A[i], z, 0, 0, 0, 127, 0, 127);
        ac[i][j][0] = fmaf(d[0], san[i] * sbm[j].x, ac[i][j][0]);
        ac[i][j][1] = fmaf(d[1], san[i] * sbm[j].y, ac[i][j][1]);
        ac[i][j][2] = fmaf(d[2], san[i] * sbm[j].z, ac[i][j][2]);
        ac[i][j][3] = fmaf(d[3], san[i] * sbm[j].w, ac[i][j][3]);
      }
    }
  };

  for (int ch = 0; ch < nch; ++ch) {
    const int64_t p = p0 + (int64_t)ch * kTile;
    const int64_t g = p / kTile;
    if constexpr (SHARE == 2) {
      v8i A[4];
      float san[4];
      load_a(at, sa, p, g, A, san);
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        v8i B[kWJ];
        float4 sbm[kWJ];
        load_b(wm + pass * kWgM, p, g, B, sbm);
        mma(A, san, B, sbm, pass ? acc2 : acc);
      }
    } else {
      v8i B[kWJ];
      float4 sbm[kWJ];
      load_b(wm, p, g, B, sbm);
#pragma unroll
      for (int pass = 0; pass < (SHARE == 1 ? 2 : 1); ++pass) {
        v8i A[4];
        float san[4];
        load_a(pass ? at2 : at, pass ? sa2 : sa, p, g, A, san);
        mma(A, san, B, sbm, pass ? acc2 : acc);
      }
    }
  }
  wgrad_store(out + (int64_t)e * NA * NB, NB, wn, wm, lr, lg, acc);
  if constexpr (SHARE == 1) wgrad_store(out2 + (int64_t)e * NA * NB, NB, wn, wm, lr, lg, acc2);
  if constexpr (SHARE == 2) wgrad_store(out + (int64_t)e * NA * NB, NB, wn, wm + kWgM, lr, lg, acc2);
}

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of the FFN backward.
struct BwdLayout {
  size_t plan, dyq, dys, xgs, fa, fb, fdh, q3, s3, poff, chunk_e, dyt, dyts, xt, xts, ht, hts,
      gt, gts, ut, uts, total;
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
                                           const float* topk_gate, float* dy, float* dgate,
                                           void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > 0x7fffffff) return MOE_ERR_SHAPE;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!dout || !y_rows || !row_of || !topk_gate || !dy || !dgate) return MOE_ERR_NULL;
  const int64_t n_rows = T * (cfg->top_k + cfg->n_shared);
  hipStream_t s = as_stream(stream);
  if (yt == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd_kernel<uint16_t>, dim3((unsigned)T), dim3(256), 0, s, dout,
                       static_cast<const uint16_t*>(y_rows), row_of, topk_gate, T, cfg->hidden,
                       cfg->top_k, cfg->n_shared, n_rows, dy, dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3((unsigned)T), dim3(256), 0, s, dout,
                       static_cast<const float*>(y_rows), row_of, topk_gate, T, cfg->hidden,
                       cfg->top_k, cfg->n_shared, n_rows, dy, dgate);
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
    hipLaunchKernelGGL(route_bwd_dx_kernel<float>, dim3((unsigned)T), dim3(256), 0, s, dl, topk_idx,
                       w_router, N, k, H, dx);
  }
  const dim3 g((unsigned)((H + 255) / 256), (unsigned)N);
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
  if (rt == MOE_BF16)
    hipLaunchKernelGGL(unpermute_sum_kernel<uint16_t>, dim3((unsigned)T), dim3(256), 0, s,
                       static_cast<const uint16_t*>(rows), row_of, extra, T, cfg->hidden, cfg->top_k,
                       cfg->n_shared, n_rows, out);
  else
    hipLaunchKernelGGL(unpermute_sum_kernel<float>, dim3((unsigned)T), dim3(256), 0, s,
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
    const float* w2ts, const uint8_t* w13t, const float* w13ts, const float* dy, void* dx_rows,
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
      H > 16384 || 2 * I > 16384)
    return MOE_ERR_UNSUPPORTED;
  if (!offsets || !dw1 || !dw3 || !dw2) return MOE_ERR_NULL;
  if (n_rows > 0 && (!row_token || !w1 || !w1s || !w3 || !w3s || !w2t || !w2ts || !w13t || !w13ts ||
                     !dy || !dx_rows))
    return MOE_ERR_NULL;
  if (n_tokens > 0 && (!xq || !xs || !x)) return MOE_ERR_NULL;
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
  const int64_t P = L.pstride, G = L.max_chunks;
  moe_status r;
  hipLaunchKernelGGL(pad_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, n_experts, (int)G, poff,
                     chunk_e);
  if (n_rows > 0) {
    r = ffn_plan_launch(offsets, n_experts, n_rows, plan, s);
    if (r != MOE_OK) return r;
    // dgrad of the down projection and the recomputed gate/up inputs (K = H)
    const int64_t it = n_rows * (I / kTile);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)n_rows), dim3(256), 0, s, dy, row_token,
                       n_rows, (int)H, dyq, dys);
    if ((r = ffn_recompute_launch(plan, n_experts, n_rows, n_tokens, xq, xs, row_token, w1, w1s, w3,
                                  w3s, (int)H, (int)I, xgs, fa, fb, s)) != MOE_OK)
      return r;
    if ((r = ffn_grouped_gemm_launch(plan, n_experts, n_rows, dyq, dys, w2t, w2ts, (int)I, (int)H, fdh,
                                     MOE_F32, s)) != MOE_OK)
      return r;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((it + 3) / 4)), dim3(256), 0, s, fa, fb, fdh,
                       n_rows, (int)I, q3, s3);
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
    hipLaunchKernelGGL((quant_tokens_kernel<float, 2>), gh, dim3(256), 0, s, dy, n_rows, n_rows, row_token,
                       offsets, poff, chunk_e, (int)H, P, dyt, dyts);
    if (xt == MOE_BF16)
      hipLaunchKernelGGL((quant_tokens_kernel<uint16_t, 1>), gh, dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), n_tokens, n_rows, row_token, offsets, poff, chunk_e,
                         (int)H, P, xtt, xts);
    else
      hipLaunchKernelGGL((quant_tokens_kernel<float, 1>), gh, dim3(256), 0, s,
                         static_cast<const float*>(x), n_tokens, n_rows, row_token, offsets, poff, chunk_e,
                         (int)H, P, xtt, xts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fdh, n_rows, n_rows, row_token,
                       offsets, poff, chunk_e, (int)I, P, htt, hts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fa, n_rows, n_rows, row_token,
                       offsets, poff, chunk_e, (int)I, P, gtt, gts);
    hipLaunchKernelGGL((quant_tokens_kernel<float, 0>), gi, dim3(256), 0, s, fb, n_rows, n_rows, row_token,
                       offsets, poff, chunk_e, (int)I, P, utt, uts);
  }
  // wgrad GEMMs (every expert's gradient written; zero for an expert without rows)
  // grid: 8 XCDs x ceil(groups / 8) groups x tiles per group
  auto wgrid = [&](int64_t NA, int64_t NB, int64_t span) {
    const int64_t groups = (NA / kTile) * n_experts;
    return dim3((unsigned)(8 * ((groups + 7) / 8) * (NB / span)));
  };
  // dW2 pairs adjacent column tiles when I allows (I % 256 == 0)
  const bool pair = I % (2 * kWgM) == 0;
  if (dwt == MOE_F32) {
    if (pair)
      hipLaunchKernelGGL((wgrad_kernel<float, 2>), wgrid(H, I, 2 * kWgM), dim3(256), 0, s, dyt, dyts,
                         nullptr, nullptr, htt, hts, poff, n_experts, (int)H, (int)I, P,
                         static_cast<float*>(dw2), nullptr);
    else
      hipLaunchKernelGGL((wgrad_kernel<float, 0>), wgrid(H, I, kWgM), dim3(256), 0, s, dyt, dyts, nullptr,
                         nullptr, htt, hts, poff, n_experts, (int)H, (int)I, P, static_cast<float*>(dw2),
                         nullptr);
    hipLaunchKernelGGL((wgrad_kernel<float, 1>), wgrid(I, H, kWgM), dim3(256), 0, s, gtt, gts, utt, uts,
                       xtt, xts, poff, n_experts, (int)I, (int)H, P, static_cast<float*>(dw1),
                       static_cast<float*>(dw3));
  } else {
    if (pair)
      hipLaunchKernelGGL((wgrad_kernel<uint16_t, 2>), wgrid(H, I, 2 * kWgM), dim3(256), 0, s, dyt, dyts,
                         nullptr, nullptr, htt, hts, poff, n_experts, (int)H, (int)I, P,
                         static_cast<uint16_t*>(dw2), nullptr);
    else
      hipLaunchKernelGGL((wgrad_kernel<uint16_t, 0>), wgrid(H, I, kWgM), dim3(256), 0, s, dyt, dyts,
                         nullptr, nullptr, htt, hts, poff, n_experts, (int)H, (int)I, P,
                         static_cast<uint16_t*>(dw2), nullptr);
    hipLaunchKernelGGL((wgrad_kernel<uint16_t, 1>), wgrid(I, H, kWgM), dim3(256), 0, s, gtt, gts, utt, uts,
                       xtt, xts, poff, n_experts, (int)I, (int)H, P, static_cast<uint16_t*>(dw1),
                       static_cast<uint16_t*>(dw3));
  }
  return launch_status();
}
