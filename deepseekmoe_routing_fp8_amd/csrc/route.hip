// Router of the DeepSeekMoE layer (2kiu.com digest section 3.2 pseudocode: sigmoid
// affinities, top-k on affinity + bias, gates normalised from the unbiased affinities,
// bincount load; section 3.4: group/node-limited routing; lpnh.cn guide section 3:
// norm_topk_prob, routed_scaling_factor, moe_gating kept out of FP8).
//
// Precision: the router weight W_r (FP32) is stored as three bf16 planes with
// W_r = hi + mid + lo exactly (moe_pack_router_weights, once per weight load). A bf16
// activation is one piece; an FP32 activation is split into three the same way. Every
// MFMA product of two bf16 pieces is exact in FP32, so the logits are sums of exact
// FP32 products; partial sums over each 128-wide K chunk are promoted into FP64.
//
// router_logits: 64 tokens x 64 experts per workgroup; the 128-K chunk of both
//   operands is staged in padded LDS and shared by 2x2 waves of 32x32 outputs.
// router_topk: one wavefront per token: ranking score s + b, optional group limit,
//   top-k in (score desc, index asc) order, gates, LDS load histogram.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// exact three-way bf16 split: v == hi + mid + lo
__device__ __forceinline__ void split3(float v, uint16_t& h, uint16_t& m, uint16_t& l) {
  h = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(h);
  m = f32_to_bf16(r1);
  l = f32_to_bf16(r1 - bf16_to_f32(m));
}

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w, int64_t n,
                                                           uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4*>(w + i);
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint16_t h[4], m[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split3(f[j], h[j], m[j], l[j]);
  *reinterpret_cast<uint2*>(out + i) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  *reinterpret_cast<uint2*>(out + n + i) = make_uint2(m[0] | ((uint32_t)m[1] << 16), m[2] | ((uint32_t)m[3] << 16));
  *reinterpret_cast<uint2*>(out + 2 * n + i) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
}

constexpr int kRT = 64, kRE = 64, kRK = 128;
constexpr int kRS = kRK + 8;      // padded LDS row (bf16 elements): 272 B, conflict-free
constexpr int kXcdsR = 8;

// XP = pieces per activation: 1 (bf16 x) or 3 (FP32 x).
template <int XP>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv, int64_t T,
                                                            int H,
                                                            const uint16_t* __restrict__ wsplit,
                                                            int N, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint16_t xl[XP][kRT][kRS];
  __shared__ __attribute__((aligned(16))) uint16_t wl[3][kRE][kRS];
  const int neb = (N + kRE - 1) / kRE;
  const int L = blockIdx.x, xcd = L % kXcdsR, slot = L / kXcdsR;
  const int64_t tb = (int64_t)(slot / neb) * kXcdsR + xcd;   // expert blocks of one token block share an XCD
  const int eb = slot % neb;
  const int64_t t0 = tb * kRT;
  if (t0 >= T) return;
  const int e0 = eb * kRE;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wt = wave >> 1, we = wave & 1;
  const int64_t NH = (int64_t)N * H;

  // global -> register staging of one K chunk
  constexpr int XSEG = XP == 1 ? 4 : 8;          // 16-byte pieces of x per thread
  uint4 xr[XSEG];
  uint4 wr[12];
  auto load = [&](int kc) {
#pragma unroll
    for (int j = 0; j < XSEG; ++j) {
      const int sidx = j * 256 + tid;
      if (XP == 1) {
        const int row = sidx >> 4, c = (sidx & 15) * 8;
        const int64_t t = min(t0 + row, T - 1);
        xr[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + t * H + kc * kRK + c);
      } else {
        const int row = sidx >> 5, c = (sidx & 31) * 4;
        const int64_t t = min(t0 + row, T - 1);
        xr[j] = *reinterpret_cast<const uint4*>(static_cast<const float*>(xv) + t * H + kc * kRK + c);
      }
    }
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int sidx = j * 256 + tid;
      const int piece = sidx >> 10, row = (sidx >> 4) & 63, c = (sidx & 15) * 8;
      const int64_t e = min(e0 + row, N - 1);
      wr[j] = *reinterpret_cast<const uint4*>(wsplit + piece * NH + e * H + kc * kRK + c);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < XSEG; ++j) {
      const int sidx = j * 256 + tid;
      if (XP == 1) {
        const int row = sidx >> 4, c = (sidx & 15) * 8;
        *reinterpret_cast<uint4*>(&xl[0][row][c]) = xr[j];
      } else {
        const int row = sidx >> 5, c = (sidx & 31) * 4;
        const float f[4] = {__uint_as_float(xr[j].x), __uint_as_float(xr[j].y),
                            __uint_as_float(xr[j].z), __uint_as_float(xr[j].w)};
        uint16_t h[4], m[4], l[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) split3(f[q], h[q], m[q], l[q]);
        *reinterpret_cast<uint2*>(&xl[0][row][c]) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        *reinterpret_cast<uint2*>(&xl[XP == 3 ? 1 : 0][row][c]) = make_uint2(m[0] | ((uint32_t)m[1] << 16), m[2] | ((uint32_t)m[3] << 16));
        *reinterpret_cast<uint2*>(&xl[XP == 3 ? 2 : 0][row][c]) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
      }
    }
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int sidx = j * 256 + tid;
      const int piece = sidx >> 10, row = (sidx >> 4) & 63, c = (sidx & 15) * 8;
      *reinterpret_cast<uint4*>(&wl[piece][row][c]) = wr[j];
    }
  };

  double acc64[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[a][b][r] = 0.0;

  const int nkc = H / kRK;
  load(0);
  store();
  __syncthreads();
  for (int kc = 0; kc < nkc; ++kc) {
    if (kc + 1 < nkc) load(kc + 1);
    v4f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kRK; ks += 32) {
      const int kk = ks + (lane >> 4) * 8;
      v8bf xa[2][XP], wb[2][3];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int p = 0; p < XP; ++p)
          xa[a][p] = *reinterpret_cast<const v8bf*>(&xl[p][wt * 32 + a * 16 + (lane & 15)][kk]);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 3; ++q)
          wb[b][q] = *reinterpret_cast<const v8bf*>(&wl[q][we * 32 + b * 16 + (lane & 15)][kk]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int p = XP - 1; p >= 0; --p)
#pragma unroll
            for (int q = 2; q >= 0; --q)   // smallest products first
              acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[a][p], wb[b][q], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc64[a][b][r] += (double)acc[a][b][r];
    __syncthreads();
    if (kc + 1 < nkc) {
      store();
      __syncthreads();
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int e = e0 + we * 32 + b * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wt * 32 + a * 16 + 4 * (lane >> 4) + r;
        if (t < T && e < N) scores[t * N + e] = (float)(1.0 / (1.0 + exp(-acc64[a][b][r])));
      }
    }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

constexpr int kTopkWaves = 4;
constexpr int kTopkTokPerWave = 4;
constexpr int kTopkTokensPerBlock = kTopkWaves * kTopkTokPerWave;
constexpr int kPerLane = kMaxRouted / kWave;  // 8 experts per lane at most

// (value desc, index asc) order: is (v, i) ahead of (bv, bi)?
__device__ __forceinline__ bool ahead(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int64_t T, int N, int k,
    int G, int Gk, int topn, float rho, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxRouted];
  __shared__ float rbuf[kTopkWaves][kMaxRouted];
  __shared__ float gbuf[kTopkWaves][kMaxGroups];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < N; i += 256) hist[i] = 0;
  __syncthreads();
  const int gsz = N / G;

  for (int it = 0; it < kTopkTokPerWave; ++it) {
    const int64_t t = ((int64_t)blockIdx.x * kTopkWaves + wave) * kTopkTokPerWave + it;
    if (t >= T) break;  // uniform per wave; no workgroup barrier inside this loop
    float sv[kPerLane], rv[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < N) {
        sv[i] = scores[t * N + e];
        rv[i] = sv[i] + bias[e];
      } else {
        sv[i] = 0.0f;
        rv[i] = -INFINITY;
      }
    }
    uint64_t keep = ~0ull;
    if (G > 1) {
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + kWave * i;
        if (e < N) rbuf[wave][e] = rv[i];
      }
      wave_lds_sync();
      float gs = -INFINITY;
      if (lane < G) {
        // sum of the topn best ranking scores of group `lane`, taken in rank order
        const float* g = &rbuf[wave][lane * gsz];
        float pv = INFINITY, sum = 0.0f;
        int pi = -1;
        for (int p = 0; p < topn; ++p) {
          float bv = -INFINITY;
          int bi = 0x7fffffff;
          for (int q = 0; q < gsz; ++q) {
            const float v = g[q];
            const bool after = v < pv || (v == pv && q > pi);
            if (after && ahead(v, q, bv, bi)) { bv = v; bi = q; }
          }
          sum = (p == 0) ? bv : sum + bv;
          pv = bv;
          pi = bi;
        }
        gs = sum;
        gbuf[wave][lane] = gs;
      }
      wave_lds_sync();
      bool kept = false;
      if (lane < G) {
        int rank = 0;
        for (int g2 = 0; g2 < G; ++g2) rank += ahead(gbuf[wave][g2], g2, gs, lane) ? 1 : 0;
        kept = rank < Gk;
      }
      keep = __ballot(kept);
      wave_lds_sync();   // rbuf/gbuf are rewritten by this wave's next token
    }
    // top-k over the experts of kept groups
    uint32_t sel = 0;
    int my_e = 0;
    float my_s = 0.0f, sum = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + kWave * i;
        if (e < N && !((sel >> i) & 1u) && ((keep >> (e / gsz)) & 1ull) && ahead(rv[i], e, bv, bi)) {
          bv = rv[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ahead(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      int win = __shfl(bi, 0);
      if (win < 0 || win >= N) win = min(j, N - 1);  // only reachable with NaN inputs
      const int owner = win & (kWave - 1), slot = win / kWave;
      float s_own = 0.0f;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) s_own = (i == slot) ? sv[i] : s_own;
      if (lane == owner) sel |= 1u << slot;
      const float sw = __shfl(s_own, owner);
      sum += sw;                         // slot order, FP32
      if (lane == j) { my_e = win; my_s = sw; }
    }
    if (lane < k) {
      idx_out[t * k + lane] = my_e;
      gate_out[t * k + lane] = __fdiv_rn(my_s, sum) * rho;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += 256)
    if (hist[i]) atomicAdd(&counts[i], hist[i]);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_pack_router_weights(const float* w_router, int64_t n_routed, int64_t hidden,
                                              uint16_t* w_split, void* stream) {
  if (n_routed < 0 || hidden <= 0 || hidden % kTile) return MOE_ERR_SHAPE;
  const int64_t n = n_routed * hidden;
  if (n == 0) return MOE_OK;
  if (!w_router || !w_split) return MOE_ERR_NULL;
  const int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 0x7fffffff) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     w_router, n, w_split);
  return launch_status();
}

extern "C" moe_status moe_route(const moe_config* cfg, const void* x, moe_dtype xt, int64_t T,
                                const uint16_t* w_router_split, const float* bias, float* scores,
                                int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (xt != MOE_F32 && xt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!counts) return MOE_ERR_NULL;
  if (T > 0 && (!x || !w_router_split || !bias || !scores || !topk_idx || !topk_gate)) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  const int N = cfg->n_routed;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((N + 255) / 256), dim3(256), 0, s, counts, N, 0);
  if (T == 0) return launch_status();
  const int64_t tblocks = (T + kRT - 1) / kRT;
  const int64_t grid = (tblocks + kXcdsR - 1) / kXcdsR * kXcdsR * ((N + kRE - 1) / kRE);
  if (grid > 0x7fffffff) return MOE_ERR_SHAPE;
  if (xt == MOE_BF16)
    hipLaunchKernelGGL(router_logits_kernel<1>, dim3((unsigned)grid), dim3(256), 0, s, x, T,
                       cfg->hidden, w_router_split, N, scores);
  else
    hipLaunchKernelGGL(router_logits_kernel<3>, dim3((unsigned)grid), dim3(256), 0, s, x, T,
                       cfg->hidden, w_router_split, N, scores);
  const unsigned g2 = (unsigned)((T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock);
  hipLaunchKernelGGL(router_topk_kernel, dim3(g2), dim3(256), 0, s, scores, bias, T, N,
                     cfg->top_k, cfg->n_group, cfg->topk_group, cfg->group_topn,
                     cfg->routed_scaling, topk_idx, topk_gate, counts);
  return launch_status();
}
