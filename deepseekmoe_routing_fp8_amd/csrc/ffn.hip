// SwiGLU experts as FP8 E4M3 grouped GEMMs with fine-grained scales (zhihu infra
// commentary, training part: E4M3 operands, 1x128 activation tiles and 128x128 weight
// blocks, the GEMM realised by promoting partial sums because the hardware has no
// matching block-scaled format; 2kiu.com digest section 4.3: accumulation kept in higher
// precision; lpnh.cn guide section 3: every GEMM input is 1x128-quantised).
//
// gfx950 design. Each 128-wide K chunk is one v_mfma_scale_f32_16x16x128_f8f6f4 with
// unit E8M0 scales (the hardware's power-of-two-per-32 scaling cannot express FP32
// scales per 128), giving an exact-product FP32 partial sum that is promoted into the
// FP32 accumulator as acc += partial * (a_scale * w_scale). The GEMM is computed
// transposed (weights are the MFMA row operand, tokens the column operand) so that a
// lane's four results share one token, hence one activation scale per chunk.
//
//   * weights stream from HBM straight into VGPRs in MFMA operand layout, several
//     chunks ahead (each weight byte is read once per M tile);
//   * the tile's activation rows (gathered through row_token) are staged in LDS with an
//     XOR swizzle, double-buffered, and shared by the 8 waves of the workgroup;
//   * a tile covers all rows of one expert up to kMT (one M tile for the usual load), so
//     the weights of an expert leave HBM once.
// Phase 1 (gate/up): wave w owns 16 intermediate columns (16 rows of W1 and the same 16
// of W3); the workgroup covers 128 columns, i.e. whole 1x128 groups of h, so the SwiGLU
// output is re-quantised in the epilogue (amax reduced across waves through LDS).
// Phase 2 (down): wave w owns 32 rows of W2; the workgroup covers 256 output features.
#include "common.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kMT = 192;              // max rows of one expert per tile (multiple of 16)
constexpr int kNTS = kMT / 16;        // MFMA column tiles per M tile
constexpr int kThreads = 512;         // 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kPD = 2;                // weight prefetch distance, in K chunks
constexpr int kMaxExperts = 1024;

struct Tile {
  int32_t e;     // expert
  int32_t m0;    // first permuted row of the tile
  int32_t mlen;  // rows in the tile (1..kMT)
  int32_t lo;    // first permuted row of the expert (identity token map)
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v8i join(const uint4& lo, const uint4& hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Tile plan: split every expert's rows into near-equal M tiles of at most kMT rows.
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int n_experts, int n_rows, int max_tiles,
                                                        Tile* __restrict__ tiles,
                                                        int32_t* __restrict__ n_tiles) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int start[kMaxExperts];
  const int e = threadIdx.x;
  int lo = 0, hi = 0, nt = 0;
  if (e < n_experts) {
    lo = min(max(offsets[e], 0), n_rows);
    hi = min(max(offsets[e + 1], lo), n_rows);
    nt = (hi - lo + kMT - 1) / kMT;
    cnt[e] = nt;
  }
  __syncthreads();
  if (e == 0) {
    int run = 0;
    for (int i = 0; i < n_experts; ++i) {
      start[i] = run;
      run += cnt[i];
    }
    *n_tiles = min(run, max_tiles);  // offsets that are not monotone cannot overflow the grid
  }
  __syncthreads();
  if (e < n_experts && nt > 0) {
    const int m = hi - lo;
    const int units = (m + 15) / 16;  // 16-row units, spread evenly over the tiles
    int row = lo;
    for (int i = 0; i < nt; ++i) {
      const int u = units / nt + (i < units % nt ? 1 : 0);
      const int len = min(u * 16, hi - row);
      if (start[e] + i < max_tiles) tiles[start[e] + i] = Tile{e, row, len, lo};
      row += len;
    }
  }
}

// Stage the 128-byte K chunk `kc` of the tile's activation rows: each thread moves 16 B.
// LDS row r holds its 8 segments at positions seg ^ (r & 7).
struct ActStage {
  uint4 v[(kMT * 8 + kThreads - 1) / kThreads];
  float s[(kMT + kThreads - 1) / kThreads];
};

__device__ __forceinline__ void act_load(ActStage& st, const uint8_t* __restrict__ aq,
                                         const float* __restrict__ as, const int* tok_s,
                                         int rows, int64_t K, int kc, int tid) {
  const int64_t nkc = K / kTile;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(st.v) / sizeof(uint4)); ++i) {
    const int slot = tid + i * kThreads;
    const int r = slot >> 3, seg = slot & 7;
    st.v[i] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const int t = tok_s[r];
      if (t >= 0) st.v[i] = *reinterpret_cast<const uint4*>(aq + (int64_t)t * K + kc * kTile + seg * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < (int)(sizeof(st.s) / sizeof(float)); ++i) {
    const int r = tid + i * kThreads;
    st.s[i] = 0.0f;
    if (r < rows) {
      const int t = tok_s[r];
      if (t >= 0) st.s[i] = as[(int64_t)t * nkc + kc];
    }
  }
}

__device__ __forceinline__ void act_store(const ActStage& st, uint8_t* act, float* scl, int rows,
                                          int tid) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(st.v) / sizeof(uint4)); ++i) {
    const int slot = tid + i * kThreads;
    const int r = slot >> 3, seg = slot & 7;
    if (r < ((rows + 15) & ~15))
      *reinterpret_cast<uint4*>(act + r * kTile + ((seg ^ (r & 7)) << 4)) = st.v[i];
  }
#pragma unroll
  for (int i = 0; i < (int)(sizeof(st.s) / sizeof(float)); ++i) {
    const int r = tid + i * kThreads;
    if (r < kMT) scl[r] = st.s[i];
  }
}

// Column operand (16 tokens x 128 K) for lane `lane` from the staged chunk: lane group g
// holds K bytes [16g, 16g+16) and [64+16g, 64+16g+16) of token (lane % 16) — the same
// K map as the weight operand, which is all the MFMA needs.
__device__ __forceinline__ v8i act_frag(const uint8_t* act, int ts, int lane) {
  const int r = ts * 16 + (lane & 15), g = lane >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(act + r * kTile + ((g ^ (r & 7)) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(act + r * kTile + (((g + 4) ^ (r & 7)) << 4));
  return join(lo, hi);
}

// Row operand: 16 weight rows x 128 K starting at `w` (row stride K), same K map.
__device__ __forceinline__ void w_load(const uint8_t* __restrict__ w, int64_t K, int kc, int lane,
                                       uint4& lo, uint4& hi) {
  const uint8_t* p = w + (int64_t)(lane & 15) * K + kc * kTile + (lane >> 4) * 16;
  const v4u a = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  const v4u b = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p + 64));
  lo = make_uint4(a[0], a[1], a[2], a[3]);
  hi = make_uint4(b[0], b[1], b[2], b[3]);
}

__device__ __forceinline__ void load_tokens(int* tok_s, const Tile& tl, const int32_t* row_token,
                                            int64_t n_tokens, int tid) {
  for (int r = tid; r < kMT; r += kThreads) {
    int t = -1;
    if (r < tl.mlen) {
      const int64_t v = row_token ? (int64_t)row_token[tl.m0 + r] : (int64_t)(tl.m0 + r - tl.lo);
      t = (v >= 0 && v < n_tokens) ? (int)v : -1;
    }
    tok_s[r] = t;
  }
}

// ------------------------------------------------------------------------------------
// Phase 1: h = silu(x W1^T) * (x W3^T), re-quantised 1x128 into hq / hs.
// grid = (max tiles, I / 128); block = 512.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ffn_gate_up_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, int64_t n_tokens,
    const int32_t* __restrict__ row_token, const uint8_t* __restrict__ w1,
    const float* __restrict__ w1s, const uint8_t* __restrict__ w3, const float* __restrict__ w3s,
    int H, int I, uint8_t* __restrict__ hq, float* __restrict__ hs) {
  __shared__ __attribute__((aligned(16))) uint8_t act[2][kMT * kTile];
  __shared__ float ascl[2][kMT];
  __shared__ int tok_s[kMT];
  __shared__ float red[kWaves][kMT];
  if ((int)blockIdx.x >= *n_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int nb = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nts = (tl.mlen + 15) >> 4;
  const int nkc = H / kTile;
  const int64_t wrow = (int64_t)nb * kTile + wave * 16;  // first W1/W3 row of this wave
  const uint8_t* wg = w1 + ((int64_t)tl.e * I + wrow) * H;
  const uint8_t* wu = w3 + ((int64_t)tl.e * I + wrow) * H;
  const float* sg_row = w1s + ((int64_t)tl.e * (I / kTile) + nb) * nkc;
  const float* su_row = w3s + ((int64_t)tl.e * (I / kTile) + nb) * nkc;

  load_tokens(tok_s, tl, row_token, n_tokens, tid);
  __syncthreads();

  uint4 wbuf[kPD + 1][4];
#pragma unroll
  for (int p = 0; p < kPD; ++p)
    if (p < nkc) {
      w_load(wg, H, p, lane, wbuf[p][0], wbuf[p][1]);
      w_load(wu, H, p, lane, wbuf[p][2], wbuf[p][3]);
    }
  ActStage st;
  act_load(st, xq, xs, tok_s, tl.mlen, H, 0, tid);
  act_store(st, act[0], ascl[0], tl.mlen, tid);
  __syncthreads();

  v4f accg[kNTS], accu[kNTS];
#pragma unroll
  for (int ts = 0; ts < kNTS; ++ts) accg[ts] = accu[ts] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kc0 = 0; kc0 < nkc; kc0 += kPD + 1) {
#pragma unroll
    for (int s = 0; s <= kPD; ++s) {
      const int kc = kc0 + s;
      if (kc < nkc) {
        const int pf = kc + kPD;                    // refill the buffer freed last step
        const int pslot = (s + kPD) % (kPD + 1);
        if (pf < nkc) {
          w_load(wg, H, pf, lane, wbuf[pslot][0], wbuf[pslot][1]);
          w_load(wu, H, pf, lane, wbuf[pslot][2], wbuf[pslot][3]);
        }
        const bool more = kc + 1 < nkc;
        if (more) act_load(st, xq, xs, tok_s, tl.mlen, H, kc + 1, tid);
        const float sbg = sg_row[kc], sbu = su_row[kc];
        const v8i ag = join(wbuf[s][0], wbuf[s][1]);
        const v8i au = join(wbuf[s][2], wbuf[s][3]);
        const uint8_t* a_lds = act[kc & 1];
        const float* s_lds = ascl[kc & 1];
#pragma unroll
        for (int ts = 0; ts < kNTS; ++ts) {
          if (ts < nts) {
            const v8i b = act_frag(a_lds, ts, lane);
            const v4f pg = mfma_fp8(ag, b);
            const v4f pu = mfma_fp8(au, b);
            const float sa = s_lds[ts * 16 + (lane & 15)];
            const float cg = sa * sbg, cu = sa * sbu;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              accg[ts][i] = fmaf(pg[i], cg, accg[ts][i]);
              accu[ts][i] = fmaf(pu[i], cu, accu[ts][i]);
            }
          }
        }
        if (more) act_store(st, act[(kc + 1) & 1], ascl[(kc + 1) & 1], tl.mlen, tid);
        __syncthreads();
      }
    }
  }

  // Epilogue: SwiGLU, amax over the 128 columns of the group, E4M3 codes.
  float h[kNTS][4];
#pragma unroll
  for (int ts = 0; ts < kNTS; ++ts) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = accg[ts][i];
      h[ts][i] = (g / (1.0f + expf(-g))) * accu[ts][i];
      m = fmaxf(m, fabsf(h[ts][i]));
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (ts < nts && lane < 16) red[wave][ts * 16 + lane] = m;
  }
  __syncthreads();
  const int nkh = I / kTile;
#pragma unroll
  for (int ts = 0; ts < kNTS; ++ts) {
    if (ts < nts) {
      const int r = ts * 16 + (lane & 15);
      float m = red[0][r];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w][r]);
      const float s = group_scale(m);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= e4m3_encode(__fdiv_rn(h[ts][i], s)) << (8 * i);
      if (r < tl.mlen) {
        const int64_t row = tl.m0 + r;
        *reinterpret_cast<uint32_t*>(hq + row * I + wrow + 4 * (lane >> 4)) = packed;
        if (wave == 0 && lane < 16) hs[row * nkh + nb] = s;
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Phase 2: y = DQ(hq) . DQ(W2)^T. grid = (max tiles, ceil(H / 256)); block = 512.
// ------------------------------------------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(kThreads) void ffn_down_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const uint8_t* __restrict__ hq, const float* __restrict__ hs, const uint8_t* __restrict__ w2,
    const float* __restrict__ w2s, int H, int I, YT* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t act[2][kMT * kTile];
  __shared__ float ascl[2][kMT];
  __shared__ int tok_s[kMT];
  if ((int)blockIdx.x >= *n_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nts = (tl.mlen + 15) >> 4;
  const int nkc = I / kTile;
  const int64_t wrow = (int64_t)blockIdx.y * 256 + wave * 32;  // first W2 row of this wave
  const bool wave_live = wrow < H;                              // H % 256 == 128 tail
  const int64_t wr_c = wave_live ? wrow : 0;
  const uint8_t* wa = w2 + ((int64_t)tl.e * H + wr_c) * I;
  const uint8_t* wb = wa + (int64_t)16 * I;
  const float* sb_row = w2s + ((int64_t)tl.e * (H / kTile) + wr_c / kTile) * nkc;

  // the hq rows of the tile are contiguous permuted rows
  for (int r = tid; r < kMT; r += kThreads) tok_s[r] = r < tl.mlen ? tl.m0 + r : -1;
  __syncthreads();

  uint4 wbuf[kPD + 1][4];
#pragma unroll
  for (int p = 0; p < kPD; ++p)
    if (p < nkc) {
      w_load(wa, I, p, lane, wbuf[p][0], wbuf[p][1]);
      w_load(wb, I, p, lane, wbuf[p][2], wbuf[p][3]);
    }
  ActStage st;
  act_load(st, hq, hs, tok_s, tl.mlen, I, 0, tid);
  act_store(st, act[0], ascl[0], tl.mlen, tid);
  __syncthreads();

  v4f acc0[kNTS], acc1[kNTS];
#pragma unroll
  for (int ts = 0; ts < kNTS; ++ts) acc0[ts] = acc1[ts] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kc0 = 0; kc0 < nkc; kc0 += kPD + 1) {
#pragma unroll
    for (int s = 0; s <= kPD; ++s) {
      const int kc = kc0 + s;
      if (kc < nkc) {
        const int pf = kc + kPD;
        const int pslot = (s + kPD) % (kPD + 1);
        if (pf < nkc) {
          w_load(wa, I, pf, lane, wbuf[pslot][0], wbuf[pslot][1]);
          w_load(wb, I, pf, lane, wbuf[pslot][2], wbuf[pslot][3]);
        }
        const bool more = kc + 1 < nkc;
        if (more) act_load(st, hq, hs, tok_s, tl.mlen, I, kc + 1, tid);
        const float sb = sb_row[kc];
        const v8i a0 = join(wbuf[s][0], wbuf[s][1]);
        const v8i a1 = join(wbuf[s][2], wbuf[s][3]);
        const uint8_t* a_lds = act[kc & 1];
        const float* s_lds = ascl[kc & 1];
#pragma unroll
        for (int ts = 0; ts < kNTS; ++ts) {
          if (ts < nts) {
            const v8i b = act_frag(a_lds, ts, lane);
            const v4f p0 = mfma_fp8(a0, b);
            const v4f p1 = mfma_fp8(a1, b);
            const float c = s_lds[ts * 16 + (lane & 15)] * sb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc0[ts][i] = fmaf(p0[i], c, acc0[ts][i]);
              acc1[ts][i] = fmaf(p1[i], c, acc1[ts][i]);
            }
          }
        }
        if (more) act_store(st, act[(kc + 1) & 1], ascl[(kc + 1) & 1], tl.mlen, tid);
        __syncthreads();
      }
    }
  }

  if (!wave_live) return;
#pragma unroll
  for (int ts = 0; ts < kNTS; ++ts) {
    const int r = ts * 16 + (lane & 15);
    if (ts < nts && r < tl.mlen) {
      YT* dst = y + (int64_t)(tl.m0 + r) * H + wrow + 4 * (lane >> 4);
      if constexpr (sizeof(YT) == 2) {
        uint2 a, b;
        a.x = f32_to_bf16(acc0[ts][0]) | ((uint32_t)f32_to_bf16(acc0[ts][1]) << 16);
        a.y = f32_to_bf16(acc0[ts][2]) | ((uint32_t)f32_to_bf16(acc0[ts][3]) << 16);
        b.x = f32_to_bf16(acc1[ts][0]) | ((uint32_t)f32_to_bf16(acc1[ts][1]) << 16);
        b.y = f32_to_bf16(acc1[ts][2]) | ((uint32_t)f32_to_bf16(acc1[ts][3]) << 16);
        *reinterpret_cast<uint2*>(dst) = a;
        *reinterpret_cast<uint2*>(dst + 16) = b;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc0[ts][0], acc0[ts][1], acc0[ts][2], acc0[ts][3]);
        *reinterpret_cast<float4*>(dst + 16) = make_float4(acc1[ts][0], acc1[ts][1], acc1[ts][2], acc1[ts][3]);
      }
    }
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
  size_t tiles, ntiles, hq, hs, total;
  int64_t max_tiles;
};

inline WsLayout ws_layout(const moe_config* c, int32_t n_experts, int64_t n_rows) {
  WsLayout L;
  L.max_tiles = (n_rows + kMT - 1) / kMT + n_experts;
  size_t off = 0;
  L.tiles = off;
  off = align256(off + (size_t)L.max_tiles * sizeof(Tile));
  L.ntiles = off;
  off = align256(off + 16);
  L.hq = off;
  off = align256(off + (size_t)n_rows * c->inter);
  L.hs = off;
  off = align256(off + (size_t)n_rows * (c->inter / kTile) * sizeof(float));
  L.total = off;
  return L;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_grouped_ffn_workspace_bytes(const moe_config* cfg, int32_t n_experts,
                                                  int64_t n_rows) {
  if (check_config(cfg) != MOE_OK || n_experts < 1 || n_rows < 0) return 0;
  return ws_layout(cfg, n_experts, n_rows).total;
}

extern "C" moe_status moe_grouped_ffn_fp8(const moe_config* cfg, int32_t n_experts, int64_t n_rows,
                                          int64_t n_tokens, const uint8_t* xq, const float* xs,
                                          const int32_t* row_token, const int32_t* offsets,
                                          const uint8_t* w1, const float* w1s, const uint8_t* w3,
                                          const float* w3s, const uint8_t* w2, const float* w2s,
                                          void* y, moe_dtype yt, void* ws, size_t ws_bytes,
                                          void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 0 || n_rows >= ((int64_t)1 << 31) ||
      n_tokens < 0 || n_tokens >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (n_rows == 0) return MOE_OK;
  if (!offsets || !w1 || !w1s || !w3 || !w3s || !w2 || !w2s || !y) return MOE_ERR_NULL;
  if (n_tokens > 0 && (!xq || !xs)) return MOE_ERR_NULL;
  const WsLayout L = ws_layout(cfg, n_experts, n_rows);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (L.max_tiles > 0x7fffffff) return MOE_ERR_SHAPE;
  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  Tile* tiles = reinterpret_cast<Tile*>(base + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(base + L.ntiles);
  uint8_t* hq = base + L.hq;
  float* hs = reinterpret_cast<float*>(base + L.hs);
  const int H = cfg->hidden, I = cfg->inter;

  hipLaunchKernelGGL(ffn_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, n_experts, (int)n_rows,
                     (int)L.max_tiles, tiles, ntiles);
  hipLaunchKernelGGL(ffn_gate_up_kernel, dim3((unsigned)L.max_tiles, I / kTile), dim3(kThreads), 0, s,
                     tiles, ntiles, xq, xs, n_tokens, row_token, w1, w1s, w3, w3s, H, I, hq, hs);
  const dim3 g2((unsigned)L.max_tiles, (unsigned)((H + 255) / 256));
  if (yt == MOE_BF16)
    hipLaunchKernelGGL(ffn_down_kernel<uint16_t>, g2, dim3(kThreads), 0, s, tiles, ntiles, hq, hs,
                       w2, w2s, H, I, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(ffn_down_kernel<float>, g2, dim3(kThreads), 0, s, tiles, ntiles, hq, hs, w2,
                       w2s, H, I, static_cast<float*>(y));
  return launch_status();
}
