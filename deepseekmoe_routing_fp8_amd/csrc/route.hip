// Router of the DeepSeekMoE layer (2kiu.com digest section 3.2 pseudocode: sigmoid
// affinities, top-k on affinity + bias, gates normalised from the unbiased affinities,
// bincount load; section 3.4: group/node-limited routing; lpnh.cn guide section 3:
// norm_topk_prob, routed_scaling_factor, moe_gating kept out of FP8).
//
// Kernel 1 (router_logits): logits = x . W_r^T on MFMA. Operands are split into bf16
// pieces whose pairwise products are exact in FP32 (x in bf16 is one piece, W_r in
// FP32 is three: hi + mid + lo == w exactly), so every product is an exact FP32
// product of the FP32 operands; partial sums over each 128-wide K chunk are promoted
// into an FP64 accumulator. Writes s = sigmoid(logit) as FP32.
// Kernel 2 (router_topk): one wavefront per token: ranking score s + b, optional group
// limit, top-k with (score desc, index asc) order, gates, LDS load histogram.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct Pieces3 {
  v8bf p[3];
};

// Split 8 FP32 values into three bf16 vectors with hi + mid + lo == v exactly.
__device__ __forceinline__ Pieces3 split3(const float (&v)[8]) {
  v8u16 h, m, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t hb = f32_to_bf16(v[i]);
    const float r1 = v[i] - bf16_to_f32(hb);
    const uint16_t mb = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mb);
    h[i] = hb;
    m[i] = mb;
    l[i] = f32_to_bf16(r2);
  }
  Pieces3 out;
  out.p[0] = __builtin_bit_cast(v8bf, h);
  out.p[1] = __builtin_bit_cast(v8bf, m);
  out.p[2] = __builtin_bit_cast(v8bf, l);
  return out;
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Block = 4 waves = 64 tokens x 64 experts; wave w: tokens t0 + 16w .. +15 (MFMA rows)
// against experts e0 .. e0+63 as four 16-column MFMA tiles.
template <bool XF32>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            int64_t T, int H,
                                                            const float* __restrict__ wr, int N,
                                                            float* __restrict__ scores) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 64;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t tok = min(t0 + row, T - 1);
  const float* wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wrow[j] = wr + (int64_t)min(e0 + 16 * j + row, N - 1) * H;

  double acc64[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[j][r] = 0.0;

  for (int kc = 0; kc < H; kc += kTile) {
    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kTile; ks += 32) {
      const int k = kc + ks + kg * 8;
      v8bf a[3];
      int na;
      if constexpr (XF32) {
        float xv8[8];
        load8(static_cast<const float*>(xv) + tok * H + k, xv8);
        const Pieces3 px = split3(xv8);
        a[0] = px.p[0]; a[1] = px.p[1]; a[2] = px.p[2];
        na = 3;
      } else {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + tok * H + k);
        a[0] = __builtin_bit_cast(v8bf, raw);
        na = 1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float wv8[8];
        load8(wrow[j] + k, wv8);
        const Pieces3 pw = split3(wv8);
        // smallest terms first
#pragma unroll
        for (int ia = 2; ia >= 0; --ia) {
          if (ia >= na) continue;
#pragma unroll
          for (int iw = 2; iw >= 0; --iw)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ia], pw.p[iw], acc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[j][r] += (double)acc[j][r];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + row;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 4 * kg + r;
      if (t < T && e < N) scores[t * N + e] = (float)(1.0 / (1.0 + exp(-acc64[j][r])));
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

constexpr int kTopkTokensPerBlock = 64;
constexpr int kPerLane = kMaxRouted / kWave;  // 8 experts per lane at most

// (value desc, index asc) order: is (v, i) ahead of (bv, bi)?
__device__ __forceinline__ bool ahead(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int64_t T, int N, int k,
    int G, int Gk, int topn, float rho, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxRouted];
  __shared__ float rbuf[4][kMaxRouted];
  __shared__ float gbuf[4][kMaxGroups];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < N; i += 256) hist[i] = 0;
  __syncthreads();
  const int gsz = N / G;
  const int64_t tbase = (int64_t)blockIdx.x * kTopkTokensPerBlock;

  for (int it = 0; it < kTopkTokensPerBlock / 4; ++it) {
    const int64_t t = tbase + it * 4 + wave;
    const bool active = t < T;  // uniform per wave
    float sv[kPerLane], rv[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + kWave * i;
      if (active && e < N) {
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
      __syncthreads();
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
      __syncthreads();
      bool kept = false;
      if (lane < G) {
        int rank = 0;
        for (int g2 = 0; g2 < G; ++g2) rank += ahead(gbuf[wave][g2], g2, gs, lane) ? 1 : 0;
        kept = rank < Gk;
      }
      keep = __ballot(kept);
    }
    // top-k over the experts of kept groups
    uint32_t sel = 0;
    int chosen[kMaxTopK];
    float chosen_s[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      chosen[j] = 0;
      chosen_s[j] = 0.0f;
      if (j >= k) continue;
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
      chosen[j] = win;
      chosen_s[j] = __shfl(s_own, owner);
    }
    if (active) {
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) sum += chosen_s[j];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k && lane == j) {
          idx_out[t * k + j] = chosen[j];
          gate_out[t * k + j] = __fdiv_rn(chosen_s[j], sum) * rho;
          atomicAdd(&hist[chosen[j]], 1);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += 256)
    if (hist[i]) atomicAdd(&counts[i], hist[i]);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const moe_config* cfg, const void* x, moe_dtype xt, int64_t T,
                                const float* w_router, const float* bias, float* scores,
                                int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T > (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (xt != MOE_F32 && xt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!counts) return MOE_ERR_NULL;
  if (T > 0 && (!x || !w_router || !bias || !scores || !topk_idx || !topk_gate)) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  const int N = cfg->n_routed;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((N + 255) / 256), dim3(256), 0, s, counts, N, 0);
  if (T == 0) return launch_status();
  const dim3 g1((unsigned)((T + 63) / 64), (unsigned)((N + 63) / 64));
  if (xt == MOE_BF16)
    hipLaunchKernelGGL(router_logits_kernel<false>, g1, dim3(256), 0, s, x, T, cfg->hidden,
                       w_router, N, scores);
  else
    hipLaunchKernelGGL(router_logits_kernel<true>, g1, dim3(256), 0, s, x, T, cfg->hidden,
                       w_router, N, scores);
  const unsigned g2 = (unsigned)((T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock);
  hipLaunchKernelGGL(router_topk_kernel, dim3(g2), dim3(256), 0, s, scores, bias, T, N,
                     cfg->top_k, cfg->n_group, cfg->topk_group, cfg->group_topn,
                     cfg->routed_scaling, topk_idx, topk_gate, counts);
  return launch_status();
}
