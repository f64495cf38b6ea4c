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
// router_logits: a workgroup (8 waves) computes a 128-expert x 128-token tile over one
//   of S contiguous ranges of K chunks (split K, so that small batches still fill the
//   chip) and writes FP64 partial logits. Operands reach LDS by direct global->LDS
//   copies in MFMA fragment order: W_r is stored pre-packed that way, x is gathered 16
//   bytes per lane. A 4-deep ring of 32-wide K steps keeps three steps in flight.
//   Workgroups with the same (K range, expert block) run on one XCD, so their W_r
//   slice (1.4 MB at the V3 shape) stays in that XCD's L2.
// router_reduce (long splits only, i.e. few tokens): one thread per (token, expert) sums
//   the S partials in a fixed order and applies the sigmoid.
// router_topk: one wavefront per token: for short splits sums the S partials itself,
//   ranking score s + b, optional group limit (each expert's rank inside its group),
//   top-k by wave-wide maxima of (score, index) keys, gates; for few tokens it also
//   counts the selections with global atomics.
// router_counts (many tokens): load histogram from topk_idx (LDS histogram per
//   workgroup, then one global atomic per expert and workgroup).
#include <algorithm>

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

__device__ __forceinline__ uint4 pack8(const uint16_t* p) {
  return make_uint4(p[0] | ((uint32_t)p[1] << 16), p[2] | ((uint32_t)p[3] << 16),
                    p[4] | ((uint32_t)p[5] << 16), p[6] | ((uint32_t)p[7] << 16));
}

constexpr int kFragElems = 512;   // one 16 x 32 bf16 MFMA operand fragment (1 KB)

// Packed W_r: plane q, expert block b16 (16 experts), K step ks (32 wide) is one
// fragment at element ((q * nb16 + b16) * (H / 32) + ks) * 512; lane l's 8 elements
// (16 bytes at l * 16) are W_q[16*b16 + l%16][32*ks + 8*(l/16) .. +8]. Experts past N
// are zero. One thread writes one lane's 8 elements of all three planes.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w, int N,
                                                           int H, int nb16,
                                                           uint16_t* __restrict__ out) {
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (b16, ks, lane)
  const int nks = H / 32;
  const int64_t per_plane = (int64_t)nb16 * nks * 64;
  if (item >= per_plane) return;
  const int lane = (int)(item & 63);
  const int64_t fr = item >> 6;                 // b16 * nks + ks
  const int b16 = (int)(fr / nks), ks = (int)(fr % nks);
  const int e = 16 * b16 + (lane & 15), k0 = 32 * ks + 8 * (lane >> 4);
  uint16_t h[8], m[8], l[8];
  if (e < N) {
    const float4 a = *reinterpret_cast<const float4*>(w + (int64_t)e * H + k0);
    const float4 b = *reinterpret_cast<const float4*>(w + (int64_t)e * H + k0 + 4);
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) split3(f[j], h[j], m[j], l[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = m[j] = l[j] = 0;
  }
  const int64_t off = item * 8;
  *reinterpret_cast<uint4*>(out + off) = pack8(h);
  *reinterpret_cast<uint4*>(out + per_plane * 8 + off) = pack8(m);
  *reinterpret_cast<uint4*>(out + 2 * per_plane * 8 + off) = pack8(l);
}

// FP32 activations -> three bf16 planes [3][T][H] (row-major), exact split.
__global__ __launch_bounds__(256) void x_split_kernel(const float* __restrict__ x, int64_t n,
                                                      uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const float4 a = *reinterpret_cast<const float4*>(x + i);
  const float4 b = *reinterpret_cast<const float4*>(x + i + 4);
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint16_t h[8], m[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) split3(f[j], h[j], m[j], l[j]);
  *reinterpret_cast<uint4*>(out + i) = pack8(h);
  *reinterpret_cast<uint4*>(out + n + i) = pack8(m);
  *reinterpret_cast<uint4*>(out + 2 * n + i) = pack8(l);
}

// ------------------------------------------------------------------------------------
// Logits
// ------------------------------------------------------------------------------------
constexpr int kLT = 128, kLE = 128;   // tokens, experts per workgroup tile
constexpr int kLThreads = 512;        // 8 waves: wave w owns experts 32*(w%4).. and tokens 64*(w/4)..
constexpr int kXcdsR = 8;
constexpr int kFragBytesR = 1024;

struct RouteGeom {
  int ntb, neb, S, n_combo, per;   // per > 0: XCDs per combination (n_combo < 8)
  int64_t grid;
};

// Split factor and launch geometry. S contiguous ranges of 128-wide K chunks are chosen
// so that there are about 256 workgroups; (range, expert block) combinations are kept
// at a divisor or a multiple of the XCD count so every XCD has work of one combination.
inline RouteGeom route_geom(int64_t T, int N, int H) {
  RouteGeom g;
  g.ntb = (int)((T + kLT - 1) / kLT);
  g.neb = (N + kLE - 1) / kLE;
  const int nkc = H / kTile;
  const int64_t tiles = (int64_t)g.ntb * g.neb;
  int S = (int)std::min<int64_t>(nkc, std::max<int64_t>(1, (256 + tiles - 1) / tiles));
  while (S * g.neb < kXcdsR && kXcdsR % (S * g.neb) != 0 && S < nkc) ++S;
  g.S = S;
  g.n_combo = S * g.neb;
  if (g.n_combo >= kXcdsR) {
    g.per = 0;
    g.grid = (int64_t)kXcdsR * ((g.n_combo + kXcdsR - 1) / kXcdsR) * g.ntb;
  } else {
    g.per = kXcdsR / g.n_combo;
    g.grid = (int64_t)kXcdsR * ((g.ntb + g.per - 1) / g.per);
  }
  return g;
}

// s_waitcnt immediate: at most n vector-memory operations outstanding, all LDS done
constexpr int waitcnt_vm_lgkm0_r(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0070; }

typedef __attribute__((address_space(3))) void lds_void_r;

__device__ __forceinline__ void dma16r(const void* g, void* lds_wave) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_r*)lds_wave, 16, 0, 0);
}

__device__ __forceinline__ v8bf lds_frag(const uint8_t* p) {
  return *reinterpret_cast<const v8bf*>(p);
}

// XP = bf16 pieces per activation: 1 (bf16 x) or 3 (FP32 x, pre-split into planes).
// Workgroup 0 also zeroes the N load counters, which the launches after this one add to
// (one launch fewer than a separate fill).
template <int XP>
__global__ __launch_bounds__(kLThreads) void router_logits_kernel(
    const uint16_t* __restrict__ xp, int64_t T, int H, const uint16_t* __restrict__ wpk, int N,
    int nb16, RouteGeom g, double* __restrict__ part, int32_t* __restrict__ counts) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < N; i += kLThreads) counts[i] = 0;
  constexpr int kXB = XP * 8 * kFragBytesR;   // x fragments per step: XP planes x 8 token blocks
  constexpr int kStage = kXB + 3 * 8 * kFragBytesR;
  constexpr int NST = XP == 1 ? 4 : 2;        // ring depth (steps in flight: NST - 1)
  constexpr int D = XP + 3;                   // copies per wave per step
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[NST > 2 ? kStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[NST > 2 ? kStage : 16];

  const int L = blockIdx.x, xcd = L % kXcdsR, slot = L / kXcdsR;
  int combo, tb;
  if (g.per == 0) {
    combo = xcd + kXcdsR * (slot / g.ntb);
    tb = slot % g.ntb;
  } else {
    if (xcd >= g.per * g.n_combo) return;
    combo = xcd % g.n_combo;
    tb = xcd / g.n_combo + g.per * slot;
  }
  if (combo >= g.n_combo || tb >= g.ntb) return;
  const int sp = combo / g.neb, eb = combo % g.neb;
  const int nkc = H / kTile;
  const int c0 = (int)((int64_t)sp * nkc / g.S), c1 = (int)((int64_t)(sp + 1) * nkc / g.S);
  const int ks0 = 4 * c0, nsteps = 4 * (c1 - c0);
  const int64_t t0 = (int64_t)tb * kLT;
  const int e0 = eb * kLE;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nks = H / 32;

  // copy sources: x fragment (plane p, token block `wave`), W fragment (plane q, expert
  // block `wave`); every lane's source stays inside the tensors (clamped rows/blocks)
  const int64_t tx = std::min<int64_t>(t0 + 16 * wave + (lane & 15), T - 1);
  const uint16_t* xsrc = xp + tx * H + 8 * (lane >> 4);
  const int64_t TH = T * H;
  const int wb16 = std::min(e0 / 16 + wave, nb16 - 1);
  const int64_t plane_elems = (int64_t)nb16 * nks * kFragElems;
  const uint16_t* wsrc = wpk + (int64_t)wb16 * nks * kFragElems + lane * 8;

  auto issue = [&](int s, uint8_t* st) {
    const int ks = ks0 + s;
#pragma unroll
    for (int p = 0; p < XP; ++p)
      dma16r(xsrc + p * TH + ks * 32, st + (p * 8 + wave) * kFragBytesR);
#pragma unroll
    for (int q = 0; q < 3; ++q)
      dma16r(wsrc + q * plane_elems + (int64_t)ks * kFragElems,
             st + kXB + (q * 8 + wave) * kFragBytesR);
  };

  const int we = 2 * (wave & 3), wt = 4 * (wave >> 2);   // first expert / token block
  v4f acc[2][4];
  double acc64[2][4][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[a][b][r] = 0.0;
    }

  auto compute = [&](const uint8_t* st) {
    v8bf wa[2][3], xb[4][XP];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 3; ++q) wa[a][q] = lds_frag(st + kXB + (q * 8 + we + a) * kFragBytesR + lane * 16);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int p = 0; p < XP; ++p) xb[b][p] = lds_frag(st + (p * 8 + wt + b) * kFragBytesR + lane * 16);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int q = 2; q >= 0; --q)   // smallest products first
#pragma unroll
          for (int p = XP - 1; p >= 0; --p)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a][q], xb[b][p], acc[a][b], 0, 0, 0);
  };

#define ROUTE_ST(S) ((S) % NST == 0 ? st0 : (S) % NST == 1 ? st1 : (S) % NST == 2 ? st2 : st3)
  // prologue: steps 0 .. NST-2 in flight
  issue(0, st0);
  if (NST > 2) {
    issue(std::min(1, nsteps - 1), st1);
    issue(std::min(2, nsteps - 1), st2);
  }
#define ROUTE_STEP(S)                                                                     \
  {                                                                                       \
    asm volatile("" ::: "memory");                                                        \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0_r((NST - 2) * D));                        \
    __builtin_amdgcn_s_barrier();                                                         \
    asm volatile("" ::: "memory");                                                        \
    issue(std::min(s0 + (S) + NST - 1, nsteps - 1), ROUTE_ST((S) + NST - 1));             \
    compute(ROUTE_ST(S));                                                                 \
  }
  for (int s0 = 0; s0 < nsteps; s0 += 4) {   // one 128-wide K chunk per iteration
    ROUTE_STEP(0) ROUTE_STEP(1) ROUTE_STEP(2) ROUTE_STEP(3)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc64[a][b][r] += (double)acc[a][b][r];
        acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
      }
  }
#undef ROUTE_STEP
#undef ROUTE_ST
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0_r(0));
  asm volatile("" ::: "memory");

  // partial logits: lane holds experts 4*(lane/16)+r of its block, token lane%16
  double* dst = part + (int64_t)sp * T * N;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t t = t0 + 16 * (wt + b) + (lane & 15);
      const int e = e0 + 16 * (we + a) + 4 * (lane >> 4);
      if (t >= T) continue;
      double* o = dst + t * N + e;
      if (e + 3 < N && (N & 1) == 0) {
        *reinterpret_cast<double2*>(o) = make_double2(acc64[a][b][0], acc64[a][b][1]);
        *reinterpret_cast<double2*>(o + 2) = make_double2(acc64[a][b][2], acc64[a][b][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) o[r] = acc64[a][b][r];
      }
    }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Affinities: one thread per (token, expert) sums the S partial logits in split order in
// FP64, applies the sigmoid and rounds to FP32. Eight partials are loaded before any is
// added, so a long split (small T: many K ranges) is not one load latency per range.
__global__ __launch_bounds__(256) void router_reduce_kernel(const double* __restrict__ part,
                                                            int S, int64_t T, int N,
                                                            float* __restrict__ scores) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * N) return;
  const int64_t plane = T * N;
  double z = 0.0;
  for (int s0 = 0; s0 < S; s0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s0 + u < S ? part[(int64_t)(s0 + u) * plane + i] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) z += v[u];
  }
  scores[i] = (float)(1.0 / (1.0 + exp(-z)));
}

// ------------------------------------------------------------------------------------
// Top-k
// ------------------------------------------------------------------------------------
constexpr int kTopkWaves = 4;
constexpr int kFusedSplits = 8;   // up to this many K ranges the top-k waves sum them
constexpr int kPerLane = kMaxRouted / kWave;  // 8 experts per lane at most

// (value desc, index asc) order: is (v, i) ahead of (bv, bi)?
__device__ __forceinline__ bool ahead(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// 64-bit key whose unsigned order is the (value desc, index asc) order; 0 = no expert
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over the wavefront (uniform result): butterflies inside each row of 16 lanes
// (quad_perm xor 1, xor 2, row_half_mirror, row_mirror), then the four rows.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp64<0xB1>(v);  v = o > v ? o : v;   // quad_perm [1,0,3,2]
  o = dpp64<0x4E>(v);  v = o > v ? o : v;   // quad_perm [2,3,0,1]
  o = dpp64<0x141>(v); v = o > v ? o : v;   // row_half_mirror
  o = dpp64<0x140>(v); v = o > v ? o : v;   // row_mirror
  uint64_t m = readlane64(v, 0);
  const uint64_t m1 = readlane64(v, 16), m2 = readlane64(v, 32), m3 = readlane64(v, 48);
  m = m1 > m ? m1 : m;
  m = m2 > m ? m2 : m;
  m = m3 > m ? m3 : m;
  return m;
}

// FUSED: the wave also sums its token's partial logits (short splits, large T);
// otherwise the affinities come from router_reduce_kernel.
template <bool FUSED>
__global__ __launch_bounds__(kTopkWaves * kWave) void router_topk_kernel(
    const double* __restrict__ part, int S, float* __restrict__ scores,
    const float* __restrict__ bias, int64_t T, int N, int k, int G, int Gk, int topn, float rho,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, int32_t* __restrict__ counts) {
  __shared__ float rbuf[kTopkWaves][kMaxRouted];
  __shared__ float gtop[kTopkWaves][kMaxRouted];
  __shared__ float gbuf[kTopkWaves][kMaxGroups];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTopkWaves + wave;
  if (t >= T) return;   // whole wave; no workgroup barrier below
  const int gsz = N / G;

  // affinities (FP64 sum of the partial logits in split order, sigmoid, rounded to FP32)
  // and bias-adjusted selection scores
  float sv[kPerLane], rv[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + kWave * i;
    sv[i] = 0.0f;
    rv[i] = -INFINITY;
    if (e < N) {
      if (FUSED) {
        double z = 0.0;
        for (int s = 0; s < S; ++s) z += part[((int64_t)s * T + t) * N + e];
        sv[i] = (float)(1.0 / (1.0 + exp(-z)));
        scores[t * N + e] = sv[i];
      } else {
        sv[i] = scores[t * N + e];
      }
      rv[i] = sv[i] + bias[e];
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
    // rank of each expert inside its group; the topn best record their scores by rank
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < N) {
        const int grp = e / gsz, base = grp * gsz;
        int rank = 0;
        for (int q = 0; q < gsz; ++q) rank += ahead(rbuf[wave][base + q], base + q, rv[i], e) ? 1 : 0;
        if (rank < topn) gtop[wave][grp * topn + rank] = rv[i];
      }
    }
    wave_lds_sync();
    float gs = -INFINITY;
    if (lane < G) {
      gs = gtop[wave][lane * topn];
      for (int p = 1; p < topn; ++p) gs += gtop[wave][lane * topn + p];   // rank order, FP32
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
  }

  uint64_t key[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + kWave * i;
    key[i] = (e < N && ((keep >> (e / gsz)) & 1ull)) ? rank_key(rv[i], e) : 0ull;
  }
  int my_e = 0;
  float my_s = 0.0f, sum = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    int win = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (best == 0 || win < 0 || win >= N) win = std::min(j, N - 1);   // only with NaN inputs
    const int owner = win & (kWave - 1), slot = win / kWave;
    float s_own = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if (i == slot) {
        s_own = sv[i];
        if (lane == owner) key[i] = 0;
      }
    }
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_own), owner));
    sum += sw;                         // slot order, FP32
    if (lane == j) {
      my_e = win;
      my_s = sw;
    }
  }
  if (lane < k) {
    idx_out[t * k + lane] = my_e;
    gate_out[t * k + lane] = __fdiv_rn(my_s, sum) * rho;
    if (counts) atomicAdd(&counts[my_e], 1);   // per-expert load (counts zeroed beforehand)
  }
}

// counts[e] += number of entries of idx equal to e (counts zeroed beforehand): per-block
// LDS histograms, then one global add per expert and block
__global__ __launch_bounds__(256) void router_counts_kernel(const int32_t* __restrict__ idx,
                                                            int64_t n, int N,
                                                            int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxRouted];
  for (int i = threadIdx.x; i < N; i += 256) hist[i] = 0;
  __syncthreads();
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += (int64_t)gridDim.x * 256) {
    const int e = idx[p];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += 256)
    if (hist[i]) atomicAdd(&counts[i], hist[i]);
}

// Up to this many selections the top-k waves count them with global atomics; beyond, the
// contention on the N counters costs more than a histogram launch.
constexpr int64_t kAtomicCountPairs = 4096;

inline size_t align256r(size_t v) { return (v + 255) & ~(size_t)255; }

struct RouteWs {
  size_t part, xsplit, total;
};

inline RouteWs route_ws(const moe_config* c, int64_t T, moe_dtype xt) {
  RouteWs w;
  const RouteGeom g = route_geom(T, c->n_routed, c->hidden);
  w.part = 0;
  w.xsplit = align256r((size_t)g.S * T * c->n_routed * sizeof(double));
  w.total = w.xsplit + (xt == MOE_F32 ? align256r((size_t)3 * T * c->hidden * 2) : 0);
  return w;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_weights_elems(int64_t n_routed, int64_t hidden) {
  if (n_routed < 1 || hidden <= 0 || hidden % kTile) return 0;
  return (size_t)3 * ((n_routed + 15) / 16 * 16) * hidden;
}

extern "C" moe_status moe_pack_router_weights(const float* w_router, int64_t n_routed, int64_t hidden,
                                              uint16_t* w_split, void* stream) {
  if (n_routed < 1 || n_routed > kMaxRouted || hidden <= 0 || hidden % kTile ||
      hidden > ((int64_t)1 << 24))
    return MOE_ERR_SHAPE;
  if (!w_router || !w_split) return MOE_ERR_NULL;
  const int nb16 = (int)((n_routed + 15) / 16);
  const int64_t items = (int64_t)nb16 * (hidden / 32) * 64;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                     as_stream(stream), w_router, (int)n_routed, (int)hidden, nb16, w_split);
  return launch_status();
}

extern "C" size_t moe_route_workspace_bytes(const moe_config* cfg, int64_t T, moe_dtype xt) {
  if (check_config(cfg) != MOE_OK || T < 0 || (xt != MOE_F32 && xt != MOE_BF16)) return 0;
  if (T == 0) return 0;
  return route_ws(cfg, T, xt).total;
}

extern "C" moe_status moe_route(const moe_config* cfg, const void* x, moe_dtype xt, int64_t T,
                                const uint16_t* w_router_split, const float* bias, float* scores,
                                int32_t* topk_idx, float* topk_gate, int32_t* counts, void* ws,
                                size_t ws_bytes, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (T < 0 || T * cfg->hidden >= ((int64_t)1 << 40) || T * cfg->top_k >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (xt != MOE_F32 && xt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!counts) return MOE_ERR_NULL;
  if (T > 0 && (!x || !w_router_split || !bias || !scores || !topk_idx || !topk_gate))
    return MOE_ERR_NULL;
  if (T > 0 && ((uintptr_t)x % 16 != 0 || (uintptr_t)w_router_split % 16 != 0))
    return MOE_ERR_UNSUPPORTED;
  const RouteWs W = route_ws(cfg, T, xt);
  if (T > 0 && (!ws || ws_bytes < W.total)) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int N = cfg->n_routed, H = cfg->hidden;
  if (T == 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3((N + 255) / 256), dim3(256), 0, s, counts, N, 0);
    return launch_status();
  }
  const RouteGeom g = route_geom(T, N, H);
  if (g.grid > 0x7fffffff || (T * N + 255) / 256 > 0x7fffffff) return MOE_ERR_SHAPE;
  uint8_t* base = static_cast<uint8_t*>(ws);
  double* part = reinterpret_cast<double*>(base + W.part);
  const int nb16 = (N + 15) / 16;
  if (xt == MOE_BF16) {
    hipLaunchKernelGGL(router_logits_kernel<1>, dim3((unsigned)g.grid), dim3(kLThreads), 0, s,
                       static_cast<const uint16_t*>(x), T, H, w_router_split, N, nb16, g, part,
                       counts);
  } else {
    uint16_t* xs3 = reinterpret_cast<uint16_t*>(base + W.xsplit);
    const int64_t n = T * H;
    hipLaunchKernelGGL(x_split_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), n, xs3);
    hipLaunchKernelGGL(router_logits_kernel<3>, dim3((unsigned)g.grid), dim3(kLThreads), 0, s,
                       xs3, T, H, w_router_split, N, nb16, g, part, counts);
  }
  // few tokens: many K ranges, summed by one thread per (token, expert) first
  const bool fused = g.S <= kFusedSplits;
  if (!fused)
    hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((T * N + 255) / 256)), dim3(256), 0,
                       s, part, g.S, T, N, scores);
  hipLaunchKernelGGL(fused ? router_topk_kernel<true> : router_topk_kernel<false>,
                     dim3((unsigned)((T + kTopkWaves - 1) / kTopkWaves)), dim3(kTopkWaves * kWave),
                     0, s, part, g.S, scores, bias, T, N, cfg->top_k, cfg->n_group, cfg->topk_group,
                     cfg->group_topn, cfg->routed_scaling, topk_idx, topk_gate,
                     T * cfg->top_k <= kAtomicCountPairs ? counts : nullptr);
  const int64_t pairs = T * cfg->top_k;
  if (pairs > kAtomicCountPairs) {
    const int cblocks = (int)std::min<int64_t>(256, (pairs + 1023) / 1024);
    hipLaunchKernelGGL(router_counts_kernel, dim3(cblocks), dim3(256), 0, s, topk_idx, pairs, N,
                       counts);
  }
  return launch_status();
}
