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
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "ffn_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kMT = 192;              // max rows of one expert per tile (multiple of 16)
constexpr int kMTShort = 160;         // tile height when segments are short (and the bound
                                      // on the tile count: every plan uses >= 160-row tiles)
constexpr int kMTMx = 160;            // power-of-two variant: 12 tiles of it would spill

// Tile height of a call: 192 rows when the segments average 192 rows or more (a tile's
// weights are streamed once per M tile, so taller tiles cut the weight traffic of long
// segments: measured 6% faster on the V3 gate/up at 16384 tokens, and at 2048 tokens of
// the width-2048 layer, 248 rows per expert, one tile per routed expert instead of two
// took the step from 0.335 to 0.300 ms), else 160 (at about 140 rows per expert the
// shared expert's taller tiles only add compute where the launch is balanced).
inline int tile_rows(int64_t n_rows, int32_t n_experts, bool mx) {
  return !mx && n_rows >= 192 * (int64_t)n_experts ? kMT : kMTShort;
}
constexpr int kMaxExperts = 1024;

struct Tile {
  int32_t e;     // expert
  int32_t m0;    // first permuted row of the tile
  int32_t mlen;  // rows in the tile (1..the call's tile height <= kMT)
  int32_t lo;    // first permuted row of the expert (identity token map)
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// Power-of-two scale variant: the MFMA applies the E8M0 block scales itself (A: the
// weight block's, uniform over the fragment; B: lane l carries the scale of column
// l % 16, the token, for its K block l / 16 - every block of the chunk has the same) and
// accumulates into c in FP32 across K, so no partial sum needs promoting.
__device__ __forceinline__ v4f mfma_fp8_scaled(const v8i& a, const v8i& b, const v4f& c, int ea,
                                               int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}


// Tile plan: split every expert's rows into near-equal M tiles of at most mt rows and
// order the experts by descending row count (ties: lower index first), so the longest
// tiles start first and the short ones fill the end of the launch. n_tiles[0] is the tile
// count; n_tiles[1], with tall tiles only, the tiles of experts with two or more (they
// come first), which the GEMM kernels schedule so that an expert's tiles share its weight
// stream (wg_work).
// One block of kMaxExperts threads, thread e for expert e.
__device__ __forceinline__ void plan_tiles(const int32_t* __restrict__ offsets, int n_experts,
                                           int n_rows, int mt, int max_tiles,
                                           Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ __attribute__((aligned(16))) int len_s[kMaxExperts];
  __shared__ int nt_r[kMaxExperts];
  __shared__ int start_r[kMaxExperts];
  __shared__ int wsum[kMaxExperts / kWave];
  __shared__ int multi_s;
  const int e = threadIdx.x, lane = e & (kWave - 1), w = e / kWave;
  if (e == 0) multi_s = 0;
  int lo = 0, hi = 0, nt = 0;
  if (e < n_experts) {
    lo = min(max(offsets[e], 0), n_rows);
    hi = min(max(offsets[e + 1], lo), n_rows);
    nt = (hi - lo + mt - 1) / mt;
  }
  const int m = hi - lo;
  len_s[e] = m;
  __syncthreads();
  if (nt >= 2) atomicAdd(&multi_s, nt);
  int rank = 0;
  if (e < n_experts) {
    // four lengths per LDS read; entries past n_experts hold 0 and never count (0 > m is
    // false for m >= 0, and their index is above e)
    const int4* l4 = reinterpret_cast<const int4*>(len_s);
    const int nq = (n_experts + 3) >> 2;
#pragma unroll 8
    for (int q = 0; q < nq; ++q) {
      const int4 v = l4[q];
      const int j = 4 * q;
      rank += (v.x > m) || (v.x == m && j < e);
      rank += (v.y > m) || (v.y == m && j + 1 < e);
      rank += (v.z > m) || (v.z == m && j + 2 < e);
      rank += (v.w > m) || (v.w == m && j + 3 < e);
    }
    nt_r[rank] = nt;   // ranks are a permutation of [0, n_experts)
  }
  __syncthreads();
  // exclusive scan of the tile counts in rank order
  const int v = e < n_experts ? nt_r[e] : 0;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += u;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  start_r[e] = before + inc - v;
  if (e == kMaxExperts - 1) {
    // offsets that are not monotone cannot overflow the grid
    const int total = min(before + inc, max_tiles);
    n_tiles[0] = total;
    // the shared-weight layout pays only for long segments (tall tiles); with short ones
    // the few multi-tile experts (the shared expert at 4096 tokens) measured 2% slower
    n_tiles[1] = mt > kMTShort ? min(multi_s, total) : 0;
  }
  __syncthreads();
  if (e < n_experts && nt > 0) {
    const int units = (m + 15) / 16;  // 16-row units, spread evenly over the tiles
    const int start = start_r[rank];
    int row = lo;
    for (int i = 0; i < nt; ++i) {
      const int u = units / nt + (i < units % nt ? 1 : 0);
      const int len = min(u * 16, hi - row);
      if (start + i < max_tiles) tiles[start + i] = Tile{e, row, len, lo};
      row += len;
    }
  }
}

__global__ __launch_bounds__(kMaxExperts) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                               int n_experts, int n_rows, int mt,
                                                               int max_tiles,
                                                               Tile* __restrict__ tiles,
                                                               int32_t* __restrict__ n_tiles) {
  plan_tiles(offsets, n_experts, n_rows, mt, max_tiles, tiles, n_tiles);
}

// Activation scales of the permuted rows, chunk-major ([H/128][n_rows]): the scales of one
// K chunk for a tile's rows are then one contiguous run, copied per chunk as a few cache
// lines instead of one line per row. Rows that name no token get scale 0 (their codes are
// never used). One block per (planned tile, group of kGatherChunks K chunks), one thread
// per row; a thread's loads for the group are all issued before its stores.
constexpr int kGatherChunks = 8;

__global__ __launch_bounds__(kMT) void ffn_gather_scales_kernel(const Tile* __restrict__ tiles,
                                                                const int32_t* __restrict__ n_tiles,
                                                                int max_tiles, int n_experts,
                                                                int n_rows, const float* __restrict__ xs,
                                                                int64_t n_tokens,
                                                                const int32_t* __restrict__ row_token,
                                                                int nkc, float* __restrict__ xsp) {
  const int tile = blockIdx.x, c0 = blockIdx.y * kGatherChunks, r = threadIdx.x;
  if (tile >= min(*n_tiles, max_tiles)) return;
  const Tile tl = tiles[tile];
  if (tl.e < 0 || tl.e >= n_experts || tl.mlen < 1 || tl.mlen > kMT || tl.m0 < 0 ||
      tl.m0 > n_rows - tl.mlen || r >= tl.mlen)
    return;
  const int64_t t = row_token ? (int64_t)row_token[tl.m0 + r] : (int64_t)(tl.m0 + r - tl.lo);
  const bool ok = t >= 0 && t < n_tokens;
  float v[kGatherChunks];
#pragma unroll
  for (int u = 0; u < kGatherChunks; ++u) v[u] = (ok && c0 + u < nkc) ? xs[t * nkc + c0 + u] : 0.0f;
#pragma unroll
  for (int u = 0; u < kGatherChunks; ++u)
    if (c0 + u < nkc) xsp[(int64_t)(c0 + u) * n_rows + tl.m0 + r] = v[u];
}

// Tile plan and scale gather of a gate/up call in one launch. Block 0 plans the tiles
// (plan_tiles); blocks 1.. gather the scales of kMaxExperts permuted rows x kGatherChunks
// K chunks each, chunk-major as ffn_gather_scales_kernel. The gather needs no plan: a
// row's token is row_token[r] or, without row_token, its index inside the segment that
// holds it (segments clamped as by the plan). Rows of no segment or without a token get
// scale 0.
__global__ __launch_bounds__(kMaxExperts) void ffn_prep_kernel(
    const int32_t* __restrict__ offsets, int n_experts, int n_rows, int mt, int max_tiles,
    Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles, const float* __restrict__ xs,
    int64_t n_tokens, const int32_t* __restrict__ row_token, int nkc, float* __restrict__ xsp) {
  if (blockIdx.x == 0) {
    plan_tiles(offsets, n_experts, n_rows, mt, max_tiles, tiles, n_tiles);
    return;
  }
  const int ncg = (nkc + kGatherChunks - 1) / kGatherChunks;
  const int b = blockIdx.x - 1;
  const int c0 = (b % ncg) * kGatherChunks;
  const int64_t r = (int64_t)(b / ncg) * kMaxExperts + threadIdx.x;
  if (r >= n_rows) return;
  int64_t t;
  if (row_token) {
    t = row_token[r];
  } else {
    auto start = [&](int e) { return min(max(offsets[e], 0), n_rows); };
    int lo_e = 0, hi_e = n_experts;   // the last segment that starts at or before r
    while (hi_e - lo_e > 1) {
      const int mid = (lo_e + hi_e) >> 1;
      if (start(mid) <= r) lo_e = mid; else hi_e = mid;
    }
    const int lo = start(lo_e), hi = min(max(offsets[lo_e + 1], lo), n_rows);
    t = r >= lo && r < hi ? r - lo : -1;
  }
  const bool ok = t >= 0 && t < n_tokens;
  float v[kGatherChunks];
  static_assert(kGatherChunks == 8, "two 16-byte loads");
  if (ok && (nkc & 3) == 0 && c0 + kGatherChunks <= nkc && ((uintptr_t)xs & 15) == 0) {
    // the token's eight scales as two 16-byte loads (t * nkc + c0 is a multiple of 4)
    const float4* p = reinterpret_cast<const float4*>(xs + t * nkc + c0);
    const float4 x0 = p[0], x1 = p[1];
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  } else {
#pragma unroll
    for (int u = 0; u < kGatherChunks; ++u) v[u] = (ok && c0 + u < nkc) ? xs[t * nkc + c0 + u] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kGatherChunks; ++u)
    if (c0 + u < nkc) xsp[(int64_t)(c0 + u) * n_rows + r] = v[u];
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and for all LDS operations (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0070; }

// Workgroup barrier for LDS data only: waits for this wave's LDS operations but not for
// its global loads in flight (__syncthreads() would add s_waitcnt vmcnt(0) and drain the
// weight ring).
constexpr int kWaitLgkm0 = 0x000F | 0x0070 | 0xC000;   // lgkmcnt(0); vmcnt, expcnt at max
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile geometry. A workgroup of 8 waves computes 256 weight rows (16 fragments of 16
// rows) against up to kMT rows of one expert.
//   wave w: two fragments, i.e. 32 weight rows (phase 1: 16 rows of W1 and the same 16
//     of W3; phase 2: 32 rows of W2), against all of the tile's rows. Its fragments
//     stream from HBM straight into a VGPR ring; no other wave needs them, so they never
//     touch LDS.
//   the tile's activation rows and scales (gathered rows, L2-resident) are copied by all
//     8 waves into an LDS ring by direct buffer->LDS loads. One workgroup barrier per
//     pair of K chunks publishes chunks c and c+1 and frees c-2 and c-1 (a barrier per
//     chunk measured 5% slower on the V3 prefill gate/up: the waves wait for the slowest
//     one twice as often).
// Both rings have RING slots. The weights run RING-1 chunks ahead, the activation copies
// a pair ahead; a wave's loads complete in issue order, so the copies are issued before
// the weights of the chunks after them and never wait behind those. All global reads are
// buffer loads: an SGPR descriptor plus a 32-bit lane offset, and reads past a
// descriptor's range return zeros without touching memory.
constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;       // 512
constexpr int kNTS = kMT / 16;                   // 16-row tiles per M tile
constexpr int kFragBytes = 16 * kTile;           // one 16 x 128 fragment: 2 KB
constexpr int kActBytes = kMT * kTile;           // activation codes per chunk (24 KB)
constexpr int kActRound = kFThreads * 16;        // bytes one copy instruction per wave moves
constexpr int kActDma = (kActBytes + kActRound - 1) / kActRound;   // copies per lane (3)
constexpr int kScaleWaves = (kMT + kWave - 1) / kWave;             // waves copying scales
constexpr int kScaleBytes = kScaleWaves * kWave * 4;
constexpr int kAStage = kActBytes + kScaleBytes; // one ring slot, a multiple of 128 bytes
constexpr int kJunk = 1024;                      // landing area of copies past the slot
constexpr int kStepOps = 4 + kActDma + 1;        // vector-memory ops per wave per chunk
constexpr int kMaxRing = 5;   // ring slots (depth 4) + the epilogue staging slot
constexpr int kMaxNbPerWg = 4;                   // n-blocks one workgroup runs back to back
constexpr int kNbPerWg1 = 2, kNbPerWg2 = 4;      // gate/up (16 blocks at I = 2048), down

// n-blocks per gate/up workgroup: one with tall tiles (measured 1.7% faster on the V3
// gate/up at 16384 skewed tokens: twice the workgroups balance the long launch better),
// else two (the same at 4096 tokens; four measured 2-4% slower everywhere), and one again
// when two would leave under four rounds of workgroups for the chip (2048 tokens at width
// 2048, 64 + 2 experts, when that layer ran 160-row tiles: 2.4 rounds with two, gate/up
// 160 -> 152 us with one; at the V3 prefill, 8.8 rounds, one measured 2.5% slower).
// Tiles: at least n_rows / tile-rows, and about one per expert when the rows spread over
// all of them.
inline int gate_up_nb_per(int64_t n_rows, int32_t n_experts, bool mx, int n_nb) {
  const int rows = tile_rows(n_rows, n_experts, mx);
  if (rows == kMT) return 1;
  const int64_t tiles = std::max<int64_t>(n_rows / rows, std::min<int64_t>(n_rows, n_experts));
  return tiles * ((n_nb + kNbPerWg1 - 1) / kNbPerWg1) < 4 * 256 ? 1 : kNbPerWg1;
}

// n-blocks per down-projection workgroup: with a few rows per expert (decode) each
// workgroup streams weights for little compute, and one block per workgroup balances the
// launch better (measured 9% faster at 4.5 rows per expert, 2-8% slower from ~140 up).
// Fewer blocks per workgroup also when n_nb blocks leave under eight rounds of workgroups
// for the chip (with at least n_rows / tile-rows tiles): with N = I (the backward's dh)
// four blocks per workgroup left 2.2 rounds, the last one mostly idle.
inline int down_nb_per(int64_t n_rows, int32_t n_experts, int n_nb) {
  int nbp = n_rows < 32 * (int64_t)n_experts ? 1 : kNbPerWg2;
  const int64_t tiles_lo = std::max<int64_t>(n_rows / tile_rows(n_rows, n_experts, false), 1);
  while (nbp > 1 && tiles_lo * ((n_nb + nbp - 1) / nbp) < 8 * 256) nbp /= 2;
  return nbp;
}
constexpr int kXcds = 8;
constexpr int kMaxChunks = 128;                  // K <= 16384
static_assert(kAStage % 128 == 0, "slot bases keep bit 6 of the swizzled offsets");
static_assert((kMaxRing - 2) * kStepOps + kStepOps <= 63, "vmcnt holds every copy in flight");

struct FfnArgs {
  const Tile* tiles;
  const int32_t* n_tiles;
  int max_tiles, n_experts, n_rows;
  const uint8_t* aq;     // activation codes: xq (phase 1) or hq (phase 2)
  const float* as;       // their 1x128 scales, chunk-major per permuted row: [K/128][n_rows]
  int64_t n_tokens;      // rows of aq
  const int32_t* row_token;
  const uint8_t* wa;     // packed W1 (phase 1) or W2 (phase 2)
  const float* wsa;
  const uint8_t* wb;     // packed W3 (phase 1)
  const float* wsb;
  int H, I, n_nb;        // n-blocks per tile
  int nb_per;            // n-blocks per workgroup (1..kMaxNbPerWg)
  uint8_t* hq;           // phase 1 outputs
  float* hs;
  void* y;               // phase 2 output; phase 3: a = x W1^T (FP32)
  float* y2;             // phase 3: b = x W3^T (FP32)
};

// Activation rows in a slot: row r keeps its 16-byte segment seg at position seg ^ (r&7).
// A column operand (16 rows x 128 K) gives lane l row l%16 and K bytes [16g, 16g+16)
// (g = l/16) and [64+16g, 64+16g+16), the K map of the packed weights. Tiles start at
// multiples of 16 rows, so r & 7 == l & 7: the lane's first half sits at byte
// act_lane_offset(l) of every tile and the second half at that offset ^ 64.
__device__ __forceinline__ uint32_t act_lane_offset(int lane) {
  return (lane & 15) * kTile + (((lane >> 4) ^ (lane & 7)) << 4);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const float lds_f32;

struct FfnLds {
  uint8_t* ast[kMaxRing];   // ring slots (kAStage bytes each, 128-byte aligned); the
                            // last one, never a ring slot, stages phase-1 h codes
  uint8_t* junk;            // kJunk bytes
  int* tok_s;               // source row of every tile row (-1: none)
  float* wsc;               // [n-block][2][kMaxChunks + kMaxRing] weight-block scales
  float* red;               // [kFWaves][kMT] phase-1 amax partials
  uint8_t* ystage;          // phase 2, bf16 output: [kMT/2][512 bytes] block rows (the
                            // last slot, enlarged)
};

// A wave-uniform pointer in scalar registers (buffer descriptors must be uniform; the
// compiler cannot always prove it for values loaded from memory).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// Weight fragment of one lane. The whole offset is in the VGPR operand: the descriptor's
// range check covers it (not an SGPR offset), so chunks past the range read zeros.
__device__ __forceinline__ v8i buf_wfrag(__amdgpu_buffer_rsrc_t d, int voff) {
  const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(d, voff, 0, 0));
  const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(d, voff + kFragBytes / 2, 0, 0));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A workgroup's set-up values, loaded into registers by ffn_kernel: the source row of
// tile row tid (a token in phase 1, a permuted row in phase 2; -1: none) and this
// thread's share of the weight-block scales of its n-blocks (entry c = tid + u * threads
// of the [n-block][2][kWscRow] table). ffn_main stores them to LDS after it has issued
// the first chunk's weight loads, so the two latencies overlap.
constexpr int kWscRowAll = kMaxChunks + kMaxRing;
constexpr int kWscPer = (kMaxNbPerWg * 2 * kWscRowAll + kFThreads - 1) / kFThreads;
struct Setup {
  int tok;
  float w[kWscPer];
};

// ------------------------------------------------------------------------------------
// Main loop and epilogue of one workgroup, for NT 16-row tiles (a compile-time count:
// the tile's rows rounded up to 16 or more; rows past the tile are computed on a clamped
// row and dropped) and a RING-slot pipeline. The K loop runs over the chunk count rounded
// up to RING and is unrolled by RING, so ring slots are static, no step computes
// conditionally and every wait is the same immediate; chunks past the last one read
// zero weights (and carry weight scales 0), adding exact zeros.
// ------------------------------------------------------------------------------------
template <int PHASE, typename YT, int NT, int RING, bool MX>
__device__ __forceinline__ void ffn_main(const FfnArgs& a, const Tile& tl, int nb0, int nbn,
                                         int wave, int lane, const FfnLds& sh, const Setup& su) {
  static_assert(RING >= 3 && RING <= kMaxRing, "ring depth");
  static_assert(NT * 16 <= kMT, "tile rows");
  constexpr bool GU = PHASE != 2;   // phases 1, 3 and 4: the gate/up GEMMs (W1 and W3)
  constexpr bool SWIGLU = PHASE == 1 || PHASE == 4;   // epilogue: h, re-quantised
  const int tid = wave * kWave + lane;
  const int K = GU ? a.H : a.I;
  const int nkc = K / kTile;
  const int last = nkc - 1;
  const int nsteps = (nkc + RING - 1) / RING * RING;   // steps per n-block

  // activation copies of this lane: kDma 16-byte units (rounds of 64 rows, as many as the
  // NT 16-row tiles need) and one scale
  constexpr int kDma = (NT * 16 * kTile + kActRound - 1) / kActRound;
  static_assert(kDma <= kActDma, "copy rounds");
  const __amdgpu_buffer_rsrc_t adesc =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.aq), 0, (int)(uint32_t)(a.n_tokens * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t sdesc =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.as), 0, (int)(uint32_t)((int64_t)a.n_rows * nkc * 4), 0x00020000);
  int aoff[kDma];   // set once the tile's source rows are in LDS (prologue)
  const int soff = (tl.m0 + min(tid, tl.mlen - 1)) * 4;   // permuted row of this lane's scale

  // This wave's two fragments of n-block nb: one descriptor per fragment row, formed per
  // step from the expert's base (32-bit offsets: H * I < 2^31, checked by every launch)
  const uint32_t frow = (uint32_t)nkc * kFragBytes;   // bytes of one 16-row fragment row
  const uint8_t* const wbaseA = a.wa + (int64_t)tl.e * a.H * a.I;
  const uint8_t* const wbaseB = GU ? a.wb + (int64_t)tl.e * a.H * a.I : wbaseA;
  auto wrow_of = [&](int nb) -> int {
    return GU ? nb * kTile + wave * 16 : nb * 256 + wave * 32;
  };
  auto wdesc = [&](int nb, int f) __attribute__((always_inline)) {
    const int wrow = wrow_of(nb);
    const uint8_t* fb;
    if (GU) {
      fb = (f == 0 ? wbaseA : wbaseB) + (uint32_t)(wrow / 16) * frow;
    } else {
      // H % 256 == 128: the last block is half used; its idle waves read block 0
      const uint32_t n16 = (uint32_t)(wrow < a.H ? wrow : 0) / 16;
      fb = wbaseA + (n16 + f) * frow;
    }
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(fb), 0, (int)frow, 0x00020000);
  };
  constexpr int kWscRow = kMaxChunks + kMaxRing;
  const int wsel0 = GU ? 0 : (wave >= 4 ? 1 : 0);   // scale row block of fragment 0
  const int wsel1 = GU ? 1 : wsel0;

  // A chunk's loads come in two groups: its weights (4 loads) and its activation copies
  // (kDma copies and 1 scale). Step g of n-block it loads the weights of chunk g of
  // that block; chunks past the block's last one (and blocks past the workgroup's range)
  // read zero weights. Activation copies depend on the chunk only.
  v8i W0[RING], W1[RING];
  const int wlane = lane * 16;
  auto issue_w = [&](int it, int c, int ws) __attribute__((always_inline)) {
    const bool real = it < nbn && c < nkc;
    const int nb = nb0 + min(it, nbn - 1);
    const int off = wlane + (real ? c : nkc) * kFragBytes;
    W0[ws] = buf_wfrag(wdesc(nb, 0), off);
    W1[ws] = buf_wfrag(wdesc(nb, 1), off);
  };
  auto issue_a = [&](int c, uint8_t* st) __attribute__((always_inline)) {
    const int cc = min(c, last);
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int at = j * kActRound + wave * 1024;
      uint8_t* dst = at < kActBytes ? st + at : sh.junk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(adesc, (lds_u8*)dst, 16, aoff[j], cc * kTile, 0, 0);
    }
    uint8_t* sdst = wave < kScaleWaves ? st + kActBytes + wave * kWave * 4 : sh.junk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sdesc, (lds_u8*)sdst, 4, soff, cc * a.n_rows * 4, 0, 0);
  };

  v4f acc0[NT], acc1[NT];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts) acc0[ts] = acc1[ts] = v4f{0.f, 0.f, 0.f, 0.f};

  // One persistent register per slot holds the lane's operand address; the second half
  // is that address ^ 64 and the scale address a per-lane constant away, both formed per
  // step, and tile offsets (multiples of 2 KB and 64 B) stay in the immediates.
  const uint32_t alo = act_lane_offset(lane);
  const int sdelta = (int)(kActBytes + (lane & 15) * 4) - (int)alo;
  lds_u8* pl[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    pl[r] = (lds_u8*)sh.ast[r] + alo;
    asm volatile("" : "+v"(pl[r]));   // a base register, not a folded constant
  }
  const float* wsc0 = nullptr;
  const float* wsc1 = nullptr;
  auto compute = [&](int c, int ws) __attribute__((always_inline)) {
    const v8i A0 = W0[ws];
    const v8i A1 = W1[ws];
    const float s0 = wsc0[c], s1 = wsc1[c];
    lds_u8* bl = pl[ws];
    lds_u8* bh = (lds_u8*)((uintptr_t)bl ^ 64);
    lds_u8* bs = bl + sdelta;
    auto frag = [&](int ts) __attribute__((always_inline)) {
      const v4i x = *reinterpret_cast<lds_v4i*>(bl + ts * 16 * kTile);
      const v4i y = *reinterpret_cast<lds_v4i*>(bh + ts * 16 * kTile);
      return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    if constexpr (MX) {
      // the MFMA applies the scales and accumulates, so nothing is promoted; the operands of
      // tile t+1 are read while tile t multiplies
      const int e0 = e8m0_of(s0), e1 = e8m0_of(s1);
      v8i mq[2];
      float ms[2];
      mq[0] = frag(0);
      ms[0] = *reinterpret_cast<lds_f32*>(bs);
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        if (ts + 1 < NT) {
          mq[(ts + 1) & 1] = frag(ts + 1);
          ms[(ts + 1) & 1] = *reinterpret_cast<lds_f32*>(bs + (ts + 1) * 64);
        }
        const int ea = e8m0_of(ms[ts & 1]);
        acc0[ts] = mfma_fp8_scaled(A0, mq[ts & 1], acc0[ts], e0, ea);
        acc1[ts] = mfma_fp8_scaled(A1, mq[ts & 1], acc1[ts], e1, ea);
        __builtin_amdgcn_sched_barrier(0);   // bound the live operands to two tiles
      }
      return;
    }
    // operands of tile t+2 are read while tile t+1 multiplies and tile t is promoted
    v8i bq[3];
    float sa[3];
    v4f p0[2], p1[2];
    bq[0] = frag(0);
    sa[0] = *reinterpret_cast<lds_f32*>(bs);
    if (NT > 1) {
      bq[1] = frag(1);
      sa[1] = *reinterpret_cast<lds_f32*>(bs + 64);
    }
    p0[0] = mfma_fp8(A0, bq[0]);
    p1[0] = mfma_fp8(A1, bq[0]);
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      if (ts + 2 < NT) {
        bq[(ts + 2) % 3] = frag(ts + 2);
        sa[(ts + 2) % 3] = *reinterpret_cast<lds_f32*>(bs + (ts + 2) * 64);
      }
      if (ts + 1 < NT) {
        p0[(ts + 1) & 1] = mfma_fp8(A0, bq[(ts + 1) % 3]);
        p1[(ts + 1) & 1] = mfma_fp8(A1, bq[(ts + 1) % 3]);
      }
      // the MFMAs of tile t+1 are issued before tile t is promoted (left to itself the
      // compiler promotes each tile right behind its own MFMAs and waits out their latency)
      __builtin_amdgcn_sched_barrier(0);
      const float c0 = sa[ts % 3] * s0, c1 = sa[ts % 3] * s1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[ts][i] = fmaf(p0[ts & 1][i], c0, acc0[ts][i]);
        acc1[ts][i] = fmaf(p1[ts & 1][i], c1, acc1[ts][i]);
      }
      __builtin_amdgcn_sched_barrier(0);   // bound the live operands to three tiles
    }
  };

  // Steps go in pairs (2p, 2p+1) with one workgroup barrier per pair. Weights run
  // RING-1 = 3 chunks ahead: step c issues the weights of chunk c+3 into the registers of
  // chunk c-1. Activations go a pair at a time: step 2p waits for the copies of chunks 2p
  // and 2p+1 (and the weights of 2p), meets the barrier (every wave's copies are in LDS,
  // every wave is done with 2p-2 and 2p-1), and issues the copies of 2p+2 and 2p+3 into
  // the slots of 2p-2 and 2p-1; step 2p+1 only waits for its weights. A wave's
  // vector-memory operations complete in issue order, so the issue order (weights of
  // 2p, copies of 2p and 2p+1, weights of 2p+1, weights of 2p+2, ...) makes every wait a
  // fixed count: at an even step the weights of the next two chunks stay in flight, at an
  // odd step also the copies of the next pair and the weights issued with them.
  // Every chunk's loads stay in the same order on loop entry as on the back edge, so the
  // compiler's own waits for the weight registers never ask for more than these.
  static_assert(RING == 4, "pairs of steps over a 4-slot ring");
  issue_w(0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // The set-up values were loaded before these weights, so they arrive first; they go to
  // LDS while the weights are in flight (an LDS-only barrier leaves the loads pending).
  // From here on the issue order is the one the waits below count.
  if (tid < kMT) sh.tok_s[tid] = su.tok;
#pragma unroll
  for (int u = 0; u < kWscPer; ++u) {
    const int c = tid + u * kFThreads;
    if (c < nbn * 2 * kWscRow) sh.wsc[c] = su.w[u];
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int unit = min((j * kActRound + wave * 1024 + lane * 16) / 16, kActBytes / 16 - 1);
    const int r = unit >> 3, seg = (unit & 7) ^ (r & 7);
    // rows past the tile and rows without a token read zeros (an offset at the end of
    // the range), so the padding of the last 16-row tile costs the matrix cores no
    // switching power
    const int src = sh.tok_s[r];
    aoff[j] = (int)(src >= 0 ? (uint32_t)src * (uint32_t)K + (uint32_t)(seg * 16)
                             : (uint32_t)(a.n_tokens * K));
  }
  __builtin_amdgcn_sched_barrier(0);
  issue_a(0, sh.ast[0]);
  issue_a(1, sh.ast[1]);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(0, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(0, 2, 2);
  __builtin_amdgcn_sched_barrier(0);
  // Every n-block ends with an epilogue that issues exactly kEpiStores stores per wave
  // (lanes with nothing to store are dropped by the buffer range check, never skipped),
  // behind the loads of the next block's first chunks; the first block gets as many dummy
  // stores behind the prologue. Loads and stores complete in issue order, so the waits of
  // a block's first two steps (before the next pair of copies is awaited) allow for the
  // stores behind them.
  constexpr int kStageStores = (kMT * 8 + kFThreads - 1) / kFThreads;   // 16-byte units
  constexpr int kYStores = kMT * 32 / kFThreads;   // 16-byte units of a staged output block
  static_assert(kMT * 32 % (2 * kFThreads) == 0 && kNTS % 2 == 0, "whole store rounds per half");
  constexpr int kEpiStores =
      SWIGLU ? kStageStores + 1 + (PHASE == 4 ? 2 * NT : 0)
             : (PHASE == 3 || sizeof(YT) == 4 ? 2 * NT : kYStores);
  static_assert(RING < kMaxRing, "the last LDS slot stages the epilogue");
  constexpr int kWOps = 4, kAOps = kDma + 1;           // loads per chunk: weights, copies
  static_assert(kWOps + kAOps <= kStepOps, "loads per chunk");
  constexpr int kWaitEven = 2 * kWOps;                  // weights of the next two chunks
  constexpr int kWaitOdd = 2 * kWOps + 2 * kAOps;       // + the next pair's copies
  static_assert(kWaitOdd + kEpiStores <= 63, "vmcnt range");
  {
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.as), 0, 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < kEpiStores; ++i)   // distinct offsets: stores the compiler cannot merge
      __builtin_amdgcn_raw_buffer_store_b32(0u, none, i * 256 + lane * 4, 0, 0);
  }
  auto group = [&](int it, int s0, auto first) __attribute__((always_inline)) {
#pragma unroll
    for (int S = 0; S < RING; ++S) {
      const int g = s0 + S + RING - 1;     // step whose weights are issued now
      const int nx = g >= nsteps ? 1 : 0;  // it belongs to the next n-block
      asm volatile("" ::: "memory");
      if (S % 2 == 0) {
        if (decltype(first)::value && S == 0)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWaitEven + kEpiStores));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWaitEven));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // copies of chunks s0+S+2 and s0+S+3 (the next block's chunks 0 and 1 in the
        // last group) into the slots of s0+S-2 and s0+S-1
        const int c2 = s0 + S + 2 - (s0 + S + 2 >= nsteps ? nsteps : 0);
        issue_a(c2, sh.ast[(S + 2) % RING]);
        issue_a(c2 + 1, sh.ast[(S + 3) % RING]);
      } else {
        if (decltype(first)::value && S == 1)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWaitOdd + kEpiStores));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWaitOdd));
        asm volatile("" ::: "memory");
      }
      issue_w(it + nx, g - nx * nsteps, (S + RING - 1) % RING);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0 + S, S);
    }
  };
  for (int it = 0; it < nbn; ++it) {
    const int nb = nb0 + it;
    wsc0 = sh.wsc + (it * 2 + wsel0) * kWscRow;
    wsc1 = sh.wsc + (it * 2 + wsel1) * kWscRow;
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) acc0[ts] = acc1[ts] = v4f{0.f, 0.f, 0.f, 0.f};
    group(it, 0, std::true_type{});
    for (int s0 = RING; s0 < nsteps; s0 += RING) group(it, s0, std::false_type{});

    // epilogue of n-block nb; the next block's first chunks are already in flight
    const int wrow = wrow_of(nb);
    if constexpr (PHASE == 3 || PHASE == 4) {
      // a = G and b = U as FP32 rows (phase 3: the backward's recompute; phase 4: the
      // SwiGLU inputs a training forward keeps, stored before h replaces G): this lane's
      // four values are columns col .. col+3 of the block's 128 (the packed W1/W3 row
      // order); rows past the tile fall outside the descriptors' ranges
      const int col = 32 * (wave >> 1) + 8 * (lane >> 4) + 4 * (wave & 1);
      const __amdgpu_buffer_rsrc_t adesc2 = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(static_cast<float*>(a.y) + (int64_t)tl.m0 * a.I + (int64_t)nb * kTile), 0,
          tl.mlen * a.I * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t bdesc2 = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.y2 + (int64_t)tl.m0 * a.I + (int64_t)nb * kTile), 0, tl.mlen * a.I * 4,
          0x00020000);
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int off = ((ts * 16 + (lane & 15)) * a.I + col) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc0[ts]), adesc2, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc1[ts]), bdesc2, off, 0, 0);
      }
    }
    if constexpr (SWIGLU) {
      // SwiGLU, amax over the 128 columns of the group (4 per lane, 4 lane groups, 8 waves)
      // h = silu(G) * U replaces G in acc0. silu(g) = g / (1 + 2^(-g log2 e)) with the
      // hardware exp2 and reciprocal: a relative error of a few 1e-7, far below the E4M3
      // step that h is rounded to next.
      float(*red)[kMT] = reinterpret_cast<float(*)[kMT]>(sh.red);
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int r = ts * 16 + (lane & 15);
        const bool valid = r < tl.mlen && sh.tok_s[r] >= 0;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc0[ts][i];
          const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
          const float h = g * __builtin_amdgcn_rcpf(1.0f + e) * acc1[ts][i];
          acc0[ts][i] = valid ? h : 0.0f;
          m = fmaxf(m, fabsf(acc0[ts][i]));
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 16) red[wave][r] = m;
        __builtin_amdgcn_sched_barrier(0);
      }
      lds_barrier();
      // codes of the tile's rows go through the staging slot (row r: 128 bytes, 16-byte
      // segment s at s ^ (r & 7)) and out as whole rows; rows past the tile fall outside
      // the descriptors' ranges
      const __amdgpu_buffer_rsrc_t qdesc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.hq + (int64_t)tl.m0 * a.I + (int64_t)nb * kTile), 0, tl.mlen * a.I, 0x00020000);
      const __amdgpu_buffer_rsrc_t hdesc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.hs + (int64_t)nb * a.n_rows + tl.m0), 0, tl.mlen * 4, 0x00020000);
      uint8_t* stage = sh.ast[kMaxRing - 1];
      // packed W1/W3 row order: this lane's four h values are columns col .. col+3 of the
      // block's 128
      const int col = 32 * (wave >> 1) + 8 * (lane >> 4) + 4 * (wave & 1);
      // the scales of tile 4*wave + lane/16 (waves 0..2 cover up to 12 tiles): one store
      const int ts_mine = 4 * wave + (lane >> 4);
      float s_mine = 0.0f;
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int r = ts * 16 + (lane & 15);
        {
          float m = red[0][r];
#pragma unroll
          for (int w = 1; w < kFWaves; ++w) m = fmaxf(m, red[w][r]);
          const float s = MX ? group_scale_pow2(m) : group_scale(m);
          // h / s as h * (1/s): within an ulp of the quotient, which the encoder rounds
          // and clamps to +-448 (exact for a power-of-two s)
          const float inv = MX ? inv_pow2(s) : __builtin_amdgcn_rcpf(s);
          const uint32_t packed = e4m3_pack4(acc0[ts][0] * inv, acc0[ts][1] * inv,
                                             acc0[ts][2] * inv, acc0[ts][3] * inv);
          *reinterpret_cast<uint32_t*>(stage + r * kTile + ((((col >> 4) ^ (r & 7))) << 4) + (col & 15)) =
              packed;
          s_mine = ts == ts_mine ? s : s_mine;
        }
        __builtin_amdgcn_sched_barrier(0);   // one tile's temporaries at a time
      }
      __builtin_amdgcn_raw_buffer_store_b32(
          __float_as_uint(s_mine), hdesc, ts_mine < NT ? (ts_mine * 16 + (lane & 15)) * 4 : (1 << 30), 0, 0);
      lds_barrier();   // the staged codes are complete; red is free for the next block
#pragma unroll
      for (int q = 0; q < kStageStores; ++q) {
        const int u = (q * kFWaves + wave) * kWave + lane;   // 16-byte unit: row u/8, segment u%8
        const int row = u >> 3, seg = u & 7, rr = min(row, kMT - 1);
        const v4u v = *reinterpret_cast<const v4u*>(stage + rr * kTile + ((seg ^ (rr & 7)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(v, qdesc, row * a.I + seg * 16, 0, 0);
      }
    } else if constexpr (PHASE == 2) {
      // rows past the tile fall outside the descriptor's range; the idle waves of a
      // half-used last block (H % 256 == 128) store past it as well
      const __amdgpu_buffer_rsrc_t ydesc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(static_cast<YT*>(a.y) + (int64_t)tl.m0 * a.H), 0,
          tl.mlen * a.H * (int)sizeof(YT), 0x00020000);
      // packed W2 row order: this lane's eight outputs are features wrow + 8*(lane/16) + 0..7
      // (acc0 the first four, acc1 the next four)
      const uint32_t cb =
          (uint32_t)((wrow < a.H ? (int)wrow : (1 << 28)) + 8 * (lane >> 4)) * (uint32_t)sizeof(YT);
      if constexpr (sizeof(YT) == 2) {
        // bf16: the block's rows are staged in LDS, half the tile at a time (row r: 512
        // bytes, 16-byte segment s at s ^ (r & 15)), and written as whole 512-byte row
        // pieces
        (void)cb;
        uint8_t* st = sh.ystage;
        const int sg = 4 * wave + (lane >> 4);   // this lane's segment of the 256-feature block
        const int fb = nb * 256;
        constexpr int kHalfTiles = kNTS / 2;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
          for (int ts = hf * kHalfTiles; ts < (hf + 1) * kHalfTiles && ts < NT; ++ts) {
            const int r = (ts - hf * kHalfTiles) * 16 + (lane & 15);
            const v4u u = {pack_bf16x2(acc0[ts][0], acc0[ts][1]), pack_bf16x2(acc0[ts][2], acc0[ts][3]),
                           pack_bf16x2(acc1[ts][0], acc1[ts][1]), pack_bf16x2(acc1[ts][2], acc1[ts][3])};
            *reinterpret_cast<v4u*>(st + r * 512 + ((sg ^ (r & 15)) << 4)) = u;
          }
          lds_barrier();
#pragma unroll
          for (int q = 0; q < kYStores / 2; ++q) {
            const int u = (q * kFWaves + wave) * kWave + lane;   // row u/32 of the half, segment u%32
            const int rh = u >> 5, seg = u & 31;
            const v4u v = *reinterpret_cast<const v4u*>(st + rh * 512 + ((seg ^ (rh & 15)) << 4));
            const int row = hf * kHalfTiles * 16 + rh;
            const int feat = fb + seg * 8;   // features past H (a half-used last block) are dropped
            const int off = feat < a.H ? (row * a.H + feat) * (int)sizeof(YT) : (1 << 30);
            __builtin_amdgcn_raw_buffer_store_b128(v, ydesc, off, 0, 0);
          }
          if (hf == 0) lds_barrier();   // the first half is read before the second is written
        }
      } else {
#pragma unroll
        for (int ts = 0; ts < NT; ++ts) {
          const int r = ts * 16 + (lane & 15);
          const uint32_t off = (uint32_t)(r * a.H) * (uint32_t)sizeof(YT) + cb;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc0[ts]), ydesc, (int)off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc1[ts]), ydesc, (int)(off + 16), 0, 0);
        }
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------
// One grouped-FFN GEMM phase over tiles (expert, M tile) x n-blocks.
//   PHASE 1: 128 intermediate columns per workgroup; epilogue h = silu(G) * U,
//            re-quantised 1x128 (amax over the 128 columns reduced across the 8
//            waves through LDS).
//   PHASE 2: 256 output features per workgroup.
//   PHASE 3: phase 1's GEMMs with G and U written as FP32 rows (the backward's recompute).
//   PHASE 4: phase 1, and G and U also written as FP32 rows (a training forward keeps the
//            SwiGLU inputs, so the backward recomputes only h from them).
// Workgroup L runs on XCD L % 8; the n-blocks of one M tile are consecutive on one XCD,
// so the tile's activation rows are fetched into that XCD's L2 once.
// ------------------------------------------------------------------------------------
// Work of workgroup L: M tile `tile` and its workgroup `wg` of nwg (n-blocks wg*nb_per ..).
// Workgroup L runs on XCD L % 8. When nwg is a multiple of 8, tiles of experts with
// several M tiles (the first n_tiles[1] of the plan) are laid out so that workgroup wg of
// every such tile runs on XCD wg % 8 at consecutive dispatch slots: the tiles of one
// expert then stream the same weight chunks at the same time through one L2 (the V3
// gate/up launch at 16384 tokens measured 6% faster). Other tiles, and every tile when
// nwg is not a multiple of 8 (the layout would leave XCDs idle), keep all their
// workgroups on one XCD, consecutively, so that XCD's L2 fetches the tile's activation
// rows once. Returns false for a workgroup without work.
__device__ __forceinline__ bool wg_work(const FfnArgs& a, int L, int* tile, int* wg) {
  const int nwg = (a.n_nb + a.nb_per - 1) / a.nb_per;
  const int total = min(a.n_tiles[0], a.max_tiles);
  const int multi = nwg % kXcds == 0 ? min(max(a.n_tiles[1], 0), total) : 0;
  const int G = (nwg + kXcds - 1) / kXcds;          // rows of 8 workgroups per shared tile
  const int la = kXcds * G * multi;
  if (L < la) {
    const int r = L / kXcds;
    *tile = r / G;
    *wg = (r % G) * kXcds + L % kXcds;
    return *wg < nwg;
  }
  const int lb = L - la, xcd = lb % kXcds, slot = lb / kXcds;
  *tile = multi + (slot / nwg) * kXcds + xcd;
  *wg = slot % nwg;
  return *tile < total;
}

// Grid of a GEMM launch over at most max_tiles tiles of n_rows rows with nwg workgroups
// each, enough for any split of the plan between the two layouts of wg_work: with NA
// shared-layout tiles it needs 8*G*NA + nwg*(tiles - NA + 7) workgroups, and NA < n_rows/80
// (an expert with nt >= 2 tiles holds more than 160 * (nt - 1) >= 80 * nt rows).
inline int64_t ffn_grid(int64_t max_tiles, int64_t nwg, int64_t n_rows) {
  if (nwg % kXcds != 0) return nwg * (max_tiles + kXcds);
  const int64_t G = nwg / kXcds;
  const int64_t na = std::min<int64_t>(max_tiles, n_rows / (kMTShort / 2) + 1);
  return nwg * (max_tiles + kXcds) + (kXcds * G - nwg) * na;
}

template <int PHASE, typename YT, bool MX>
__global__ __launch_bounds__(kFThreads) void ffn_kernel(const FfnArgs a) {
  __shared__ __attribute__((aligned(128))) uint8_t ast0[kAStage];
  __shared__ __attribute__((aligned(128))) uint8_t ast1[kAStage];
  __shared__ __attribute__((aligned(128))) uint8_t ast2[kAStage];
  __shared__ __attribute__((aligned(128))) uint8_t ast3[kAStage];
  // the last slot stages the epilogue: phase-1 h codes, or a phase-2 bf16 output block
  __shared__ __attribute__((aligned(128)))
  uint8_t ast4[PHASE == 2 && sizeof(YT) == 2 ? kMT / 2 * 512 : kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t junk[kJunk];
  __shared__ int tok_s[kMT];
  constexpr int kWscRow = kMaxChunks + kMaxRing;
  __shared__ float wsc[kMaxNbPerWg * 2][kWscRow];   // weight-block scales per n-block, row
                                                     // block and K chunk; 0 past the last chunk
  __shared__ float red[PHASE == 1 || PHASE == 4 ? kFWaves * kMT : 1];
  constexpr bool GU = PHASE != 2;
  int tile, wg;
  if (!wg_work(a, blockIdx.x, &tile, &wg)) return;
  const int nb0 = wg * a.nb_per;
  const int nbn = min(a.nb_per, a.n_nb - nb0);
  const Tile tl = a.tiles[tile];
  // a workspace that does not hold this call's plan must not lead out of bounds
  if (tl.e < 0 || tl.e >= a.n_experts || tl.mlen < 1 || tl.mlen > (MX ? kMTMx : kMT) || tl.m0 < 0 ||
      tl.m0 > a.n_rows - tl.mlen)
    return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = GU ? a.H : a.I;
  const int nkc = K / kTile;

  // set-up values (stored to LDS by ffn_main): the source row of tile row tid, a token
  // (phase 1) or a permuted row (phase 2), and this thread's entries of the weight-block
  // scales for every K chunk (0 past the last one) of each n-block: phase 1 (W1, W3) of
  // row block nb; phase 2 the two W2 row blocks of the block's 256 rows
  static_assert(kMT <= kFThreads && kWscRow == kWscRowAll, "one tile row per thread");
  Setup su;
  su.tok = -1;
  if (tid < tl.mlen) {
    if (GU) {
      const int64_t v = a.row_token ? (int64_t)a.row_token[tl.m0 + tid] : (int64_t)(tl.m0 + tid - tl.lo);
      su.tok = (v >= 0 && v < a.n_tokens) ? (int)v : -1;
    } else {
      su.tok = tl.m0 + tid;
    }
  }
  const int64_t nrb = (GU ? a.I : a.H) / kTile;
#pragma unroll
  for (int u = 0; u < kWscPer; ++u) {
    const int c = tid + u * kFThreads;
    const int it = c / (2 * kWscRow), which = (c / kWscRow) & 1, kc = c % kWscRow;
    const int nb = nb0 + it;
    float v = 0.0f;
    if (c >= nbn * 2 * kWscRow || kc >= nkc) {
    } else if (GU) {
      v = (which == 0 ? a.wsa : a.wsb)[((int64_t)tl.e * nrb + nb) * nkc + kc];
    } else {
      const int64_t rb = min((int64_t)nb * 2 + which, nrb - 1);
      v = a.wsa[((int64_t)tl.e * nrb + rb) * nkc + kc];
    }
    su.w[u] = v;
  }

  const FfnLds sh{{ast0, ast1, ast2, ast3, ast4}, junk, tok_s, &wsc[0][0], red, ast4};
  // Ring depth 4: three chunks (96 KB of weights per CU) in flight cover the loaded HBM
  // latency, the accumulators of 12 16-row tiles still fit beside the ring (three
  // registers spilled, reloaded only in the epilogue), and K
  // chunk counts of the usual shapes (56, 16) divide by it, so no block ends in steps
  // of zero weights. (A depth of 5 for the shorter tiles measured 1.5% slower on the
  // V3 prefill gate/up: its 60 padded steps per block cost more than the depth gained.)
  constexpr int R = 4;
  switch ((tl.mlen + 15) >> 4) {
    case 1: case 2: ffn_main<PHASE, YT, 2, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    case 3: case 4: ffn_main<PHASE, YT, 4, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    case 5: case 6: ffn_main<PHASE, YT, 6, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    case 7: case 8: ffn_main<PHASE, YT, 8, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    case 9: ffn_main<PHASE, YT, 9, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    case 10: ffn_main<PHASE, YT, 10, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su); break;
    default:
      if constexpr (!MX) ffn_main<PHASE, YT, 12, R, MX>(a, tl, nb0, nbn, wave, lane, sh, su);
      break;
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
  size_t tiles, ntiles, hq, hs, xsp, total;
  int64_t max_tiles;
};

inline WsLayout ws_layout(const moe_config* c, int32_t n_experts, int64_t n_rows) {
  WsLayout L;
  L.max_tiles = (n_rows + kMTShort - 1) / kMTShort + n_experts;
  size_t off = 0;
  L.tiles = off;
  off = align256(off + (size_t)L.max_tiles * sizeof(Tile));
  L.ntiles = off;
  off = align256(off + 16);
  L.hq = off;
  off = align256(off + (size_t)n_rows * c->inter);
  L.hs = off;
  off = align256(off + (size_t)n_rows * (c->inter / kTile) * sizeof(float));
  L.xsp = off;
  off = align256(off + (size_t)n_rows * (c->hidden / kTile) * sizeof(float));
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

namespace {

// Checks shared by the three entry points; fills the workspace pointers.
struct FfnCall {
  WsLayout L;
  Tile* tiles;
  int32_t* ntiles;
  uint8_t* hq;
  float* hs;
  float* xsp;
};

moe_status ffn_check(const moe_config* cfg, int32_t n_experts, int64_t n_rows, void* ws,
                     size_t ws_bytes, FfnCall* f) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 0 || n_rows >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (cfg->hidden > kMaxChunks * kTile || cfg->inter > kMaxChunks * kTile) return MOE_ERR_UNSUPPORTED;
  // per-lane operand offsets into hq and the chunk-major scale arrays are 32-bit
  if (n_rows * (int64_t)cfg->inter >= ((int64_t)1 << 32) ||
      n_rows * (int64_t)(cfg->hidden / kTile) * 4 >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  f->L = ws_layout(cfg, n_experts, n_rows);
  if (n_rows == 0) return MOE_OK;
  if (!ws || ws_bytes < f->L.total) return MOE_ERR_WORKSPACE;
  // total work-items of the larger launch must fit the 32-bit grid size
  const int64_t nb_max = std::max<int64_t>(cfg->inter / kTile, (cfg->hidden + 255) / 256);
  if (ffn_grid(f->L.max_tiles, nb_max, n_rows) * kFThreads >= ((int64_t)1 << 32))
    return MOE_ERR_UNSUPPORTED;
  uint8_t* base = static_cast<uint8_t*>(ws);
  f->tiles = reinterpret_cast<Tile*>(base + f->L.tiles);
  f->ntiles = reinterpret_cast<int32_t*>(base + f->L.ntiles);
  f->hq = base + f->L.hq;
  f->hs = reinterpret_cast<float*>(base + f->L.hs);
  f->xsp = reinterpret_cast<float*>(base + f->L.xsp);
  return MOE_OK;
}

// save: a training forward, which also writes the SwiGLU inputs a = G and b = U to
// a_out and b_out ([n_rows, I] FP32 each).
moe_status ffn_gate_up(const moe_config* cfg, int32_t n_experts, int64_t n_rows, int64_t n_tokens,
                       const uint8_t* xq, const float* xs, const int32_t* row_token,
                       const int32_t* offsets, const uint8_t* w1, const float* w1s,
                       const uint8_t* w3, const float* w3s, void* ws, size_t ws_bytes,
                       void* stream, bool save = false, float* a_out = nullptr,
                       float* b_out = nullptr) {
  FfnCall f;
  const moe_status st = ffn_check(cfg, n_experts, n_rows, ws, ws_bytes, &f);
  if (st != MOE_OK) return st;
  if (n_tokens < 0 || n_tokens * (int64_t)cfg->hidden >= ((int64_t)1 << 32))
    return n_tokens < 0 ? MOE_ERR_SHAPE : MOE_ERR_UNSUPPORTED;
  if (save && cfg->scale_mode != 0) return MOE_ERR_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  if (!offsets || !w1 || !w1s || !w3 || !w3s) return MOE_ERR_NULL;
  if (n_tokens > 0 && (!xq || !xs)) return MOE_ERR_NULL;
  if (save && (!a_out || !b_out)) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  const int H = cfg->hidden, I = cfg->inter;
  // plan and scale gather in one launch; also without tokens: every row's scale is then
  // written as 0, never left undefined
  const int64_t prep_blocks =
      1 + (n_rows + kMaxExperts - 1) / kMaxExperts * ((H / kTile + kGatherChunks - 1) / kGatherChunks);
  hipLaunchKernelGGL(ffn_prep_kernel, dim3((unsigned)prep_blocks), dim3(kMaxExperts), 0, s, offsets,
                     n_experts, (int)n_rows, tile_rows(n_rows, n_experts, cfg->scale_mode == 1),
                     (int)f.L.max_tiles, f.tiles, f.ntiles, xs, n_tokens, row_token, H / kTile,
                     f.xsp);
  FfnArgs a1{f.tiles, f.ntiles, (int)f.L.max_tiles, n_experts, (int)n_rows, xq, f.xsp, n_tokens,
             row_token, w1, w1s, w3, w3s, H, I, I / kTile,
             gate_up_nb_per(n_rows, n_experts, cfg->scale_mode == 1, I / kTile), f.hq, f.hs, a_out, b_out};
  const dim3 grid((unsigned)ffn_grid(f.L.max_tiles, (a1.n_nb + a1.nb_per - 1) / a1.nb_per, n_rows));
  if (save)
    hipLaunchKernelGGL((ffn_kernel<4, uint16_t, false>), grid, dim3(kFThreads), 0, s, a1);
  else if (cfg->scale_mode == 1)
    hipLaunchKernelGGL((ffn_kernel<1, uint16_t, true>), grid, dim3(kFThreads), 0, s, a1);
  else
    hipLaunchKernelGGL((ffn_kernel<1, uint16_t, false>), grid, dim3(kFThreads), 0, s, a1);
  return launch_status();
}

moe_status ffn_down(const moe_config* cfg, int32_t n_experts, int64_t n_rows, const uint8_t* w2,
                    const float* w2s, void* y, moe_dtype yt, void* ws, size_t ws_bytes,
                    void* stream) {
  FfnCall f;
  const moe_status st = ffn_check(cfg, n_experts, n_rows, ws, ws_bytes, &f);
  if (st != MOE_OK) return st;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (n_rows == 0) return MOE_OK;
  if (!w2 || !w2s || !y) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  const int H = cfg->hidden, I = cfg->inter;
  FfnArgs a2{f.tiles, f.ntiles, (int)f.L.max_tiles, n_experts, (int)n_rows, f.hq, f.hs, n_rows,
             nullptr, w2, w2s, nullptr, nullptr, H, I, (H + 255) / 256,
             down_nb_per(n_rows, n_experts, (H + 255) / 256),
             nullptr, nullptr, y};
  const dim3 grid((unsigned)ffn_grid(f.L.max_tiles, (a2.n_nb + a2.nb_per - 1) / a2.nb_per, n_rows));
  const bool mx = cfg->scale_mode == 1;
  if (yt == MOE_BF16 && mx)
    hipLaunchKernelGGL((ffn_kernel<2, uint16_t, true>), grid, dim3(kFThreads), 0, s, a2);
  else if (yt == MOE_BF16)
    hipLaunchKernelGGL((ffn_kernel<2, uint16_t, false>), grid, dim3(kFThreads), 0, s, a2);
  else if (mx)
    hipLaunchKernelGGL((ffn_kernel<2, float, true>), grid, dim3(kFThreads), 0, s, a2);
  else
    hipLaunchKernelGGL((ffn_kernel<2, float, false>), grid, dim3(kFThreads), 0, s, a2);
  return launch_status();
}

}  // namespace

// ------------------------------------------------------------------------------------
// The phase-2 kernel as a plain grouped GEMM, for the backward pass:
// y[rows, N] = A[rows, K] x W_e[N, K]^T per expert segment, on a tile plan of the same
// segments. A: E4M3 codes with 1x128 scales chunk-major ([K/128][n_rows]); W_e packed by
// moe_pack_fp8_weights with 128x128 block scales [E][N/128][K/128].
// ------------------------------------------------------------------------------------
namespace moe {

size_t ffn_plan_bytes(int32_t n_experts, int64_t n_rows) {
  const int64_t max_tiles = (n_rows + kMTShort - 1) / kMTShort + n_experts;
  return align256((size_t)max_tiles * sizeof(Tile)) + 256;
}

moe_status ffn_plan_launch(const int32_t* offsets, int32_t n_experts, int64_t n_rows, void* plan,
                           hipStream_t s) {
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 1 || n_rows >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  const int64_t max_tiles = (n_rows + kMTShort - 1) / kMTShort + n_experts;
  Tile* tiles = static_cast<Tile*>(plan);
  int32_t* nt = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(plan) +
                                           align256((size_t)max_tiles * sizeof(Tile)));
  hipLaunchKernelGGL(ffn_plan_kernel, dim3(1), dim3(kMaxExperts), 0, s, offsets, n_experts,
                     (int)n_rows, tile_rows(n_rows, n_experts, false), (int)max_tiles, tiles, nt);
  return launch_status();
}

moe_status ffn_grouped_gemm_launch(const void* plan, int32_t n_experts, int64_t n_rows,
                                   const uint8_t* aq, const float* as_cm, const uint8_t* w,
                                   const float* wsc, int N, int K, void* y, moe_dtype yt,
                                   hipStream_t s) {
  if (N <= 0 || K <= 0 || N % kTile || K % kTile || K > kMaxChunks * kTile) return MOE_ERR_SHAPE;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 1 || n_rows >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if ((int64_t)N * K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;   // 32-bit weight offsets
  // per-lane operand offsets into A and the scale array are 32-bit
  if (n_rows * (int64_t)K >= ((int64_t)1 << 32) || n_rows * (int64_t)(K / kTile) * 4 >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  const int64_t max_tiles = (n_rows + kMTShort - 1) / kMTShort + n_experts;
  const int n_nb = (N + 255) / 256;
  const int nbp = down_nb_per(n_rows, n_experts, n_nb);
  const int64_t nwg = (n_nb + nbp - 1) / nbp;
  if (ffn_grid(max_tiles, nwg, n_rows) * kFThreads >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  const Tile* tiles = static_cast<const Tile*>(plan);
  const int32_t* nt = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(plan) +
                                                       align256((size_t)max_tiles * sizeof(Tile)));
  FfnArgs a{tiles, nt, (int)max_tiles, n_experts, (int)n_rows, aq, as_cm, n_rows, nullptr, w, wsc,
            nullptr, nullptr, N, K, n_nb, nbp, nullptr, nullptr, y};
  const dim3 grid((unsigned)ffn_grid(max_tiles, nwg, n_rows));
  if (yt == MOE_BF16)
    hipLaunchKernelGGL((ffn_kernel<2, uint16_t, false>), grid, dim3(kFThreads), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_kernel<2, float, false>), grid, dim3(kFThreads), 0, s, a);
  return launch_status();
}

moe_status ffn_recompute_launch(const void* plan, int32_t n_experts, int64_t n_rows,
                                int64_t n_tokens, const uint8_t* xq, const float* xs,
                                const int32_t* row_token, const uint8_t* w1, const float* w1s,
                                const uint8_t* w3, const float* w3s, int H, int I, float* xsp,
                                float* a_out, float* b_out, hipStream_t s) {
  if (H <= 0 || I <= 0 || H % kTile || I % kTile || H > kMaxChunks * kTile) return MOE_ERR_SHAPE;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 1 || n_rows >= ((int64_t)1 << 31) ||
      n_tokens < 0)
    return MOE_ERR_SHAPE;
  if ((int64_t)H * I >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;   // 32-bit weight offsets
  // per-lane operand offsets into xq and the chunk-major scales are 32-bit
  if (n_tokens * (int64_t)H >= ((int64_t)1 << 32) || n_rows * (int64_t)(H / kTile) * 4 >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  const int64_t max_tiles = (n_rows + kMTShort - 1) / kMTShort + n_experts;
  const int n_nb = I / kTile;
  const int64_t nwg = (n_nb + kNbPerWg1 - 1) / kNbPerWg1;
  if (ffn_grid(max_tiles, nwg, n_rows) * kFThreads >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  const Tile* tiles = static_cast<const Tile*>(plan);
  const int32_t* nt = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(plan) +
                                                       align256((size_t)max_tiles * sizeof(Tile)));
  // also without tokens: every row's scale is then written as 0, never left undefined
  hipLaunchKernelGGL(ffn_gather_scales_kernel,
                       dim3((unsigned)max_tiles, (unsigned)((H / kTile + kGatherChunks - 1) / kGatherChunks)),
                       dim3(kMT), 0, s, tiles, nt, (int)max_tiles, n_experts, (int)n_rows, xs, n_tokens,
                       row_token, H / kTile, xsp);
  FfnArgs a{tiles, nt, (int)max_tiles, n_experts, (int)n_rows, xq, xsp, n_tokens, row_token, w1, w1s,
            w3, w3s, H, I, n_nb, kNbPerWg1, nullptr, nullptr, a_out, b_out};
  hipLaunchKernelGGL((ffn_kernel<3, float, false>), dim3((unsigned)ffn_grid(max_tiles, nwg, n_rows)), dim3(kFThreads), 0,
                     s, a);
  return launch_status();
}

}  // namespace moe

extern "C" moe_status moe_grouped_ffn_fp8_gate_up(const moe_config* cfg, int32_t n_experts,
                                                  int64_t n_rows, int64_t n_tokens,
                                                  const uint8_t* xq, const float* xs,
                                                  const int32_t* row_token,
                                                  const int32_t* offsets, const uint8_t* w1,
                                                  const float* w1s, const uint8_t* w3,
                                                  const float* w3s, void* ws, size_t ws_bytes,
                                                  void* stream) {
  return ffn_gate_up(cfg, n_experts, n_rows, n_tokens, xq, xs, row_token, offsets, w1, w1s, w3,
                     w3s, ws, ws_bytes, stream);
}

extern "C" moe_status moe_grouped_ffn_fp8_gate_up_train(
    const moe_config* cfg, int32_t n_experts, int64_t n_rows, int64_t n_tokens, const uint8_t* xq,
    const float* xs, const int32_t* row_token, const int32_t* offsets, const uint8_t* w1,
    const float* w1s, const uint8_t* w3, const float* w3s, float* a_out, float* b_out, void* ws,
    size_t ws_bytes, void* stream) {
  return ffn_gate_up(cfg, n_experts, n_rows, n_tokens, xq, xs, row_token, offsets, w1, w1s, w3,
                     w3s, ws, ws_bytes, stream, true, a_out, b_out);
}

extern "C" moe_status moe_grouped_ffn_fp8_down(const moe_config* cfg, int32_t n_experts,
                                               int64_t n_rows, const uint8_t* w2, const float* w2s,
                                               void* y, moe_dtype yt, void* ws, size_t ws_bytes,
                                               void* stream) {
  return ffn_down(cfg, n_experts, n_rows, w2, w2s, y, yt, ws, ws_bytes, stream);
}

extern "C" moe_status moe_grouped_ffn_fp8(const moe_config* cfg, int32_t n_experts, int64_t n_rows,
                                          int64_t n_tokens, const uint8_t* xq, const float* xs,
                                          const int32_t* row_token, const int32_t* offsets,
                                          const uint8_t* w1, const float* w1s, const uint8_t* w3,
                                          const float* w3s, const uint8_t* w2, const float* w2s,
                                          void* y, moe_dtype yt, void* ws, size_t ws_bytes,
                                          void* stream) {
  // validate both halves before launching either
  FfnCall f;
  moe_status st = ffn_check(cfg, n_experts, n_rows, ws, ws_bytes, &f);
  if (st != MOE_OK) return st;
  if (yt != MOE_BF16 && yt != MOE_F32) return MOE_ERR_DTYPE;
  if (n_rows > 0 && (!w2 || !w2s || !y)) return MOE_ERR_NULL;
  st = ffn_gate_up(cfg, n_experts, n_rows, n_tokens, xq, xs, row_token, offsets, w1, w1s, w3, w3s,
                   ws, ws_bytes, stream);
  if (st != MOE_OK) return st;
  return ffn_down(cfg, n_experts, n_rows, w2, w2s, y, yt, ws, ws_bytes, stream);
}

extern "C" moe_status moe_grouped_ffn_intermediate_offsets(const moe_config* cfg,
                                                           int32_t n_experts, int64_t n_rows,
                                                           size_t* hq_offset, size_t* hs_offset) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!hq_offset || !hs_offset) return MOE_ERR_NULL;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 0 || n_rows >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  const WsLayout L = ws_layout(cfg, n_experts, n_rows);
  *hq_offset = L.hq;
  *hs_offset = L.hs;
  return MOE_OK;
}

// ------------------------------------------------------------------------------------
// The grouped FFN without a caller-provided workspace, for callers that cannot allocate
// device memory (code under graph capture, serving loops, harnesses without hipMalloc).
// The workspace is a static device array of MOE_NOALLOC_SCRATCH_BYTES per GPU. In host
// code the array's name stands for a host-side shadow, so its device address is looked
// up once per device with that device current (hipGetSymbolAddress) and only that
// address is ever handed to a kernel. Nothing in the workspace needs clearing: the plan
// kernel writes the tile list and its count, and every row a later launch reads is
// written by an earlier one of the same call.
// ------------------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kScratchDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the device's first call).
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_grouped_ffn_fp8_noalloc(const moe_config* cfg, int32_t n_experts,
                                                  int64_t n_rows, int64_t n_tokens,
                                                  const uint8_t* xq, const float* xs,
                                                  const int32_t* row_token, const int32_t* offsets,
                                                  const uint8_t* w1, const float* w1s,
                                                  const uint8_t* w3, const float* w3s,
                                                  const uint8_t* w2, const float* w2s, void* y,
                                                  moe_dtype yt, void* stream) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (n_experts < 1 || n_experts > kMaxExperts || n_rows < 0 || n_rows >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (ws_layout(cfg, n_experts, n_rows).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_SCRATCH;
  if (n_rows == 0)   // validates the rest, launches nothing
    return moe_grouped_ffn_fp8(cfg, n_experts, 0, n_tokens, xq, xs, row_token, offsets, w1, w1s,
                               w3, w3s, w2, w2s, y, yt, nullptr, 0, stream);
  void* ws = nullptr;
  const moe_status sa = scratch_address(&ws);
  if (sa != MOE_OK) return sa;
  return moe_grouped_ffn_fp8(cfg, n_experts, n_rows, n_tokens, xq, xs, row_token, offsets, w1, w1s,
                             w3, w3s, w2, w2s, y, yt, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
