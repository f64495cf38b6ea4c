/*
 * moe_fp8.h — C ABI of a gfx950 (MI355X) library for the forward pass of a
 * DeepSeek-V3-style DeepSeekMoE layer: sigmoid routing with the auxiliary-loss-free
 * expert bias and an optional group limit, FP8 E4M3 SwiGLU experts with 1x128
 * activation tiles and 128x128 weight blocks, a shared expert, the weighted combine
 * and the sign-based bias update.
 *
 * Sources (web pages, cited by title and section):
 *   [guide]  lpnh.cn, "从技术报告到可跑配置：DeepSeek-V3 的 MoE、MLA、FP8 到底难在哪",
 *            section 3 (model JSON; [fp8] block: e4m3, tile_wise_1x128 inputs,
 *            block_wise_128x128 weights, moe_gating kept out of FP8).
 *   [digest] 2kiu.com DeepSeek-V3 technical-report digest: section 3.2 (sigmoid
 *            affinities, bias used only for ranking, normalised gates, load bincount,
 *            +-gamma update after each step), section 3.3 (sequence-level balance
 *            loss), section 3.4 (group/node-limited routing,
 *            no token dropping), section 4.3 (per-group scales, higher-precision
 *            accumulation), section 5.2 (batch-level load statistics), section 5.5 (per-sequence
 *            allocation entropy).
 *   [zhihu]  zhihu infra commentary on the report, training part (E4M3 throughout,
 *            1x128 / 128x128 groups, GEMM by partial-sum promotion; SwiGLU recompute).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers owned by the caller unless stated otherwise; a
 *     pointer to an array with zero elements may be NULL. The
 *     library never allocates, frees or keeps a pointer; scratch memory comes in
 *     through an explicit workspace whose size is queried first. The one exception is
 *     moe_grouped_ffn_fp8_noalloc, whose workspace is a static device array.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *     enqueued asynchronously; results are valid after the caller synchronises.
 *   - Arguments are validated on the host before any launch. A failed check returns
 *     the status and launches nothing. A failed launch returns MOE_ERR_HIP. No C++
 *     exception crosses this interface.
 *   - All matrices are row-major and densely packed. E4M3 codes are OCP E4M3FN bytes
 *     (the bit patterns of torch.float8_e4m3fn). bf16 is passed as uint16 bits.
 *   - NaN/Inf in inputs give unspecified values but never out-of-bounds accesses.
 *   - Calls are thread-safe and results deterministic. The only global state is the
 *     per-device address of moe_grouped_ffn_fp8_noalloc's static array (looked up once
 *     per device under a lock); concurrent calls of that entry point on one GPU race on
 *     the array itself.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MOE_ERR_SHAPE = 2,       /* a size or config field is out of range            */
  MOE_ERR_DTYPE = 3,       /* unsupported dtype for this argument               */
  MOE_ERR_UNSUPPORTED = 4, /* valid request the library does not implement       */
  MOE_ERR_HIP = 5,         /* a HIP launch or runtime call failed               */
  MOE_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the queried size   */
  MOE_ERR_SCRATCH = 7      /* request larger than the static scratch buffer of
                              moe_grouped_ffn_fp8_noalloc                          */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer configuration; field meanings follow the model JSON of [guide] section 3. */
typedef struct moe_config {
  int32_t hidden;          /* H: hidden size, multiple of 128                         */
  int32_t inter;           /* I: expert intermediate size, multiple of 128            */
  int32_t n_routed;        /* N_r: routed experts, 1..512                             */
  int32_t n_shared;        /* N_s: shared experts, 0..16                              */
  int32_t top_k;           /* k: experts per token, 1..16                             */
  int32_t n_group;         /* G: expert groups (1 disables the limit); N_r % G == 0,
                              G <= 64                                                 */
  int32_t topk_group;      /* G_k: groups a token may use, 1..G; k <= G_k * N_r / G   */
  int32_t group_topn;      /* affinities summed into a group score, 1..N_r/G          */
  float routed_scaling;    /* rho: gates of a token sum to rho ([guide] routed_scaling_factor) */
  float bias_gamma;        /* gamma: bias step ([guide] expert_bias_update_rate)      */
  int32_t scale_mode;      /* grouped FFN scales: 0 = FP32 group scales, partial sums
                              promoted in FP32 per 128-wide K chunk (the pages' scheme);
                              1 = power-of-two group scales (moe_quantize_*_pow2), applied
                              exactly by the MFMA's block-scale operands with FP32
                              accumulation across K (opt-in variant)                  */
} moe_config;

/* Human-readable text for a status (static storage). */
const char* moe_status_string(moe_status s);

/*
 * moe_quantize_1x128 — fine-grained activation quantisation ([guide] section 3
 * tile_wise_1x128, e4m3; [digest] section 4.3; [zhihu] per-tile 1x128).
 * For each row and each 128-wide column tile: amax = max|x|, scale s = fl32(amax/448)
 * (s = 1 when that is 0), code = E4M3 round-to-nearest-even of fl32(x/s), saturating
 * at +-448, sign kept.
 *   x       [rows, cols] of dtype xt (MOE_F32 or MOE_BF16)
 *   q       [rows, cols] uint8 E4M3 codes (output)
 *   scales  [rows, cols/128] float (output)
 * Errors: NULL pointers; rows < 0; cols <= 0 or cols % 128 != 0.
 */
moe_status moe_quantize_1x128(const void* x, moe_dtype xt, int64_t rows, int64_t cols,
                              uint8_t* q, float* scales, void* stream);

/*
 * moe_quantize_128x128 — weight-block quantisation, the preparation of the GEMM
 * weight operand ([guide] section 3 block_wise_128x128; [zhihu] per-group 128x128).
 * Same rule as moe_quantize_1x128 over each 128x128 block of each matrix.
 *   w       [mats, rows, cols] float
 *   q       [mats, rows, cols] uint8 (output)
 *   scales  [mats, rows/128, cols/128] float (output)
 * Errors: NULL pointers; mats < 0; rows or cols not positive multiples of 128.
 */
moe_status moe_quantize_128x128(const float* w, int64_t mats, int64_t rows, int64_t cols,
                                uint8_t* q, float* scales, void* stream);

/*
 * moe_quantize_1x128_pow2, moe_quantize_128x128_pow2 — the same groups with power-of-two
 * scales, for scale_mode 1 (an opt-in variant; the pages call the fine-grained scheme
 * close to micro-scaling, [zhihu] training part, [digest] section 4.3). A group's scale
 * is the smallest power of two s with amax / s <= 448 (s = 1 for an all-zero group,
 * s >= 2^-126); codes = E4M3 round-to-nearest-even of x / s (exact division).
 * Arguments, layouts and errors as moe_quantize_1x128 / moe_quantize_128x128.
 */
moe_status moe_quantize_1x128_pow2(const void* x, moe_dtype xt, int64_t rows, int64_t cols,
                                   uint8_t* q, float* scales, void* stream);
moe_status moe_quantize_128x128_pow2(const float* w, int64_t mats, int64_t rows, int64_t cols,
                                     uint8_t* q, float* scales, void* stream);

/*
 * moe_pack_fp8_weights — re-lays E4M3 weight codes for the grouped FFN (a byte
 * permutation, no arithmetic). The FFN streams each 16-row x 128-column fragment of a
 * weight matrix as 2 KB of contiguous memory in MFMA operand order, which HBM serves at
 * close to its sequential bandwidth. For a [rows, cols] matrix, fragment (n16, kc) sits
 * at byte ((n16 * cols/128) + kc) * 2048, as two 1 KB halves h = 0, 1; byte b of lane l
 * (0..63) in half h holds code [rho(n16, l%16)][128*kc + 64*h + 16*(l/16) + b] with
 * rho(n16, j) = 32*(n16/2) + 8*(j/4) + 4*(n16%2) + j%4: the two fragments of a 32-row
 * group interleave their rows by 4, so that the eight outputs a lane gets from the pair
 * are adjacent columns of the result.
 *   q       [mats, rows, cols] uint8 row-major codes (e.g. from moe_quantize_128x128)
 *   packed  [mats, rows*cols] uint8, output; must not overlap q
 * Errors: NULL pointers; rows % 32 or cols % 128 != 0; q == packed (UNSUPPORTED).
 */
moe_status moe_pack_fp8_weights(const uint8_t* q, int64_t mats, int64_t rows, int64_t cols,
                                uint8_t* packed, void* stream);

/*
 * moe_pack_router_weights — stores the FP32 router weight W_r as three bf16 planes
 * (hi, mid, lo) with W_r == hi + mid + lo exactly, the form moe_route reads. Done once
 * per weight load; lets the router run its FP32-exact products on bf16 MFMAs.
 * Exact for every |W_r| >= 2^-110 and 0; below that the last piece is rounded to
 * bf16's subnormal grid (error <= 2^-133).
 * Layout (MFMA fragment order): with nb16 = ceil(N_r/16), plane q (0 = RNE bf16 of W_r,
 * 1 = mid, 2 = lo), expert block b (16 experts) and K step ks (32 columns) form one
 * 512-element fragment at element ((q*nb16 + b)*(H/32) + ks)*512; its elements
 * 8*l .. 8*l+7 are plane q of W_r[16*b + l%16][32*ks + 8*(l/16) .. +8], l = 0..63.
 * Rows past N_r are zero.
 *   w_router  [N_r, H] float
 *   w_split   moe_router_weights_elems(N_r, H) bf16 bit patterns, output, 16-byte aligned
 * Errors: NULL pointers; N_r outside 1..512; H not a positive multiple of 128.
 */
moe_status moe_pack_router_weights(const float* w_router, int64_t n_routed, int64_t hidden,
                                   uint16_t* w_split, void* stream);

/* Elements of moe_pack_router_weights' output: 3 * ceil(N_r/16)*16 * H (0 if invalid). */
size_t moe_router_weights_elems(int64_t n_routed, int64_t hidden);

/*
 * moe_route — router ([digest] section 3.2 pseudocode and prose; section 3.4 group
 * limit; [guide] section 3 norm_topk_prob, routed_scaling_factor, gating kept in
 * high precision).
 *   s = sigmoid(x . W_r^T) from unquantised x. Every product is an exact product of the
 *   FP32 operands (bf16-piece MFMAs), summed in FP32 within each 128-wide K chunk and
 *   promoted into FP64 accumulators (per contiguous range of chunks, then the ranges
 *   in order); s is rounded to FP32. Ranking score s + b (FP32).
 *   With G > 1: a group's score is the FP32 sum of its group_topn best ranking scores;
 *   the G_k best groups are kept (ties: lower group index); experts elsewhere are
 *   excluded. Top-k by ranking score, descending, ties to the lower expert index.
 *   Gates: s[idx_j] / sum_j s[idx_j] * rho (unbiased s). counts[e] = selections of e.
 *   x               [T, H] of dtype xt, 16-byte aligned
 *   w_router_split  packed planes of W_r from moe_pack_router_weights
 *   bias            [N_r] float
 *   scores          [T, N_r] float, output: the sigmoid affinities s
 *   topk_idx        [T, k] int32, output, slot order = descending ranking score
 *   topk_gate       [T, k] float, output
 *   counts          [N_r] int32, output (overwritten, not accumulated)
 *   ws              workspace of moe_route_workspace_bytes(cfg, T, xt) bytes (partial
 *                   logits; NULL allowed when that is 0)
 * Errors: NULL pointers; invalid config (see moe_config); T < 0; workspace;
 * MOE_ERR_UNSUPPORTED for misaligned x or w_router_split.
 */
moe_status moe_route(const moe_config* cfg, const void* x, moe_dtype xt, int64_t T,
                     const uint16_t* w_router_split, const float* bias, float* scores,
                     int32_t* topk_idx, float* topk_gate, int32_t* counts, void* ws,
                     size_t ws_bytes, void* stream);

/* Workspace bytes moe_route needs for T tokens of dtype xt (0 for T = 0 or invalid). */
size_t moe_route_workspace_bytes(const moe_config* cfg, int64_t T, moe_dtype xt);

/*
 * moe_permute — group the (token, slot) pairs by expert ([digest] section 3.2: the
 * output sums ffn_expert[idx[j]] over the slots; section 3.4: every token reaches its
 * experts, none is dropped), followed by one segment per shared expert that every token
 * passes ([guide] section 3: num_shared_experts; [digest] section 3.2: shared plus
 * routed experts), so a single moe_grouped_ffn_fp8 call over N_r + N_s experts serves
 * both. The expert histogram is recomputed from topk_idx, so the outputs are consistent
 * with it by construction.
 *   offsets   [N_r+N_s+1] int32, output. offsets[0..N_r] is the exclusive prefix sum of
 *             the routed loads; offsets[N_r+1+s] = T*k + (s+1)*T.
 *   row_token [T*(k+N_s)] int32, output: token of each permuted row. Rows of routed
 *             expert e are offsets[e]..offsets[e+1]-1 in ascending token order; shared
 *             expert s owns rows T*k + s*T + t (token t). Rows offsets[N_r]..T*k-1 exist
 *             only when topk_idx holds entries outside [0, N_r); they carry -1 (a row the
 *             grouped FFN turns into zeros) and belong to the first shared segment.
 *   row_of    [T, k] int32, output: permuted row of (t, j)
 *   ws        workspace of moe_permute_workspace_bytes(cfg, T) bytes (NULL when 0)
 * topk_idx entries outside [0, N_r) are skipped (their row_of is -1). Experts must be
 * distinct within a token (moe_route guarantees it); otherwise rows are unspecified
 * but all accesses stay in bounds.
 * Errors: NULL pointers; invalid config; T < 0 or T*(k+N_s) >= 2^31; workspace.
 */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* row_token, int32_t* row_of, void* ws,
                       size_t ws_bytes, void* stream);

/* Workspace bytes moe_permute needs for T tokens (per-block expert counts; 0 for T = 0). */
size_t moe_permute_workspace_bytes(const moe_config* cfg, int64_t T);

/* Workspace bytes the grouped FFN needs for n_experts experts and n_rows rows (the same
 * figure serves moe_grouped_ffn_fp8 and the gate_up / down pair). */
size_t moe_grouped_ffn_workspace_bytes(const moe_config* cfg, int32_t n_experts,
                                       int64_t n_rows);

/*
 * moe_grouped_ffn_fp8 — SwiGLU experts as FP8 grouped GEMMs ([zhihu] training part:
 * E4M3 operands with 1x128 / 128x128 scales, GEMM by partial-sum promotion; SwiGLU;
 * [digest] section 4.3: higher-precision accumulation; [guide] section 3: all GEMM
 * inputs 1x128-quantised).
 * For permuted row r of expert e (offsets[e] <= r < offsets[e+1]) with token
 * t = row_token[r] (or t = r - offsets[e] when row_token is NULL):
 *   G = DQ(xq_t) . DQ(W1_e)^T, U = DQ(xq_t) . DQ(W3_e)^T — every 128-wide K chunk is one
 *   FP8 MFMA partial sum, promoted into an FP32 accumulator times a_scale * w_scale;
 *   h = silu(G) * U in FP32, with silu(g) = g * rcp(1 + exp2(-g * log2(e))) on the
 *   hardware exp2 and reciprocal (relative error a few 1e-7); then 1x128 groups of h
 *   along I: s = fl32(amax / 448) (1 when 0) as in moe_quantize_1x128, but codes =
 *   E4M3 of h * rcp(s) (within an ulp of the correctly rounded quotient that
 *   moe_quantize_1x128 uses). G and U carry FP32 accumulation differences anyway, so hq
 *   is not a bit-exact quantity: a code can differ by one E4M3 step from a reference
 *   quantisation of an exact h where h / s sits next to a rounding boundary;
 *   y_r = DQ(hq) . DQ(W2_e)^T with the same promotion, stored as yt.
 *   n_tokens  rows of xq / xs
 *   xq, xs    [n_tokens, H] uint8, [n_tokens, H/128] float
 *   row_token [n_rows] int32 or NULL
 *   offsets   [n_experts+1] int32, device; read on the device (no host sync).
 *             Values are clamped to [0, n_rows].
 *   w1, w3    [n_experts, I, H] E4M3 codes in the layout of moe_pack_fp8_weights;
 *             w1s, w3s [n_experts, I/128, H/128] float (row-major block scales)
 *   w2        [n_experts, H, I] codes, packed likewise; w2s [n_experts, H/128, I/128] float
 *   y         [n_rows, H] of dtype yt (MOE_BF16 or MOE_F32), output
 *   ws        workspace of at least moe_grouped_ffn_workspace_bytes(...) bytes; holds
 *             the tile plan and the quantised intermediate (hq, hs) between the halves
 * Rows whose token index falls outside [0, n_tokens) produce y = 0. Rows outside every
 * expert segment are not written.
 * Errors: NULL pointers; invalid config; n_experts < 1 or > 1024; n_rows < 0;
 * workspace; MOE_ERR_UNSUPPORTED for H or I > 16384, n_tokens*H or n_rows*I >= 2^32.
 * Equivalent to moe_grouped_ffn_fp8_gate_up followed by moe_grouped_ffn_fp8_down.
 */
moe_status moe_grouped_ffn_fp8(const moe_config* cfg, int32_t n_experts, int64_t n_rows,
                               int64_t n_tokens, const uint8_t* xq, const float* xs,
                               const int32_t* row_token, const int32_t* offsets,
                               const uint8_t* w1, const float* w1s, const uint8_t* w3,
                               const float* w3s, const uint8_t* w2, const float* w2s,
                               void* y, moe_dtype yt, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * moe_grouped_ffn_intermediate_offsets — where moe_grouped_ffn_fp8_gate_up (and
 * moe_grouped_ffn_fp8) leave the quantised intermediate inside the workspace, for
 * callers that read it: hq at byte *hq_offset, [n_rows, I] uint8 E4M3 codes, row-major;
 * hs at byte *hs_offset, [I/128][n_rows] float, chunk-major (the scale of row r's
 * group c is hs[c * n_rows + r]). Only rows inside the expert segments are written.
 * Host-only, launches nothing.
 * Errors: NULL outputs; invalid config; n_experts outside 1..1024 or n_rows outside
 * 0..2^31-1 (SHAPE).
 */
moe_status moe_grouped_ffn_intermediate_offsets(const moe_config* cfg, int32_t n_experts,
                                                int64_t n_rows, size_t* hq_offset,
                                                size_t* hs_offset);

/*
 * moe_grouped_ffn_fp8_gate_up — first half of moe_grouped_ffn_fp8 (same passages):
 * plans the tiles from offsets, computes G, U, h and stores its 1x128 re-quantisation
 * (hq, hs) in ws. Arguments as in moe_grouped_ffn_fp8.
 */
moe_status moe_grouped_ffn_fp8_gate_up(const moe_config* cfg, int32_t n_experts,
                                       int64_t n_rows, int64_t n_tokens, const uint8_t* xq,
                                       const float* xs, const int32_t* row_token,
                                       const int32_t* offsets, const uint8_t* w1,
                                       const float* w1s, const uint8_t* w3, const float* w3s,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn_fp8_gate_up_train — moe_grouped_ffn_fp8_gate_up for a training step: the
 * same launch and the same (hq, hs), and the SwiGLU inputs are kept for the backward
 * ([zhihu] training part: SwiGLU is among the operators recomputed in the backward, so
 * what is kept is its input, not its output h):
 *   a_out, b_out  [n_rows, I] float each, output: a = G, b = U of every row of every expert
 *                 segment (the FP32 accumulators h is formed from); rows outside every
 *                 segment are not written. moe_grouped_ffn_fp8_backward takes them as
 *                 a_saved, b_saved and then recomputes only h.
 * Errors: as moe_grouped_ffn_fp8_gate_up; NULL a_out or b_out (n_rows > 0);
 * scale_mode != 0 (UNSUPPORTED: the backward runs on the FP32 group scales only).
 */
moe_status moe_grouped_ffn_fp8_gate_up_train(const moe_config* cfg, int32_t n_experts,
                                             int64_t n_rows, int64_t n_tokens,
                                             const uint8_t* xq, const float* xs,
                                             const int32_t* row_token, const int32_t* offsets,
                                             const uint8_t* w1, const float* w1s,
                                             const uint8_t* w3, const float* w3s, float* a_out,
                                             float* b_out, void* ws, size_t ws_bytes,
                                             void* stream);

/*
 * moe_grouped_ffn_fp8_down — second half: y = DQ(hq) . DQ(W2_e)^T for every row, from
 * the plan and intermediate that the preceding moe_grouped_ffn_fp8_gate_up call with the
 * same cfg, n_experts and n_rows left in ws (stream-ordered after it). If ws holds no
 * such result, y is unspecified but every access stays in bounds.
 */
moe_status moe_grouped_ffn_fp8_down(const moe_config* cfg, int32_t n_experts, int64_t n_rows,
                                    const uint8_t* w2, const float* w2s, void* y, moe_dtype yt,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn_fp8_noalloc — moe_grouped_ffn_fp8 with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, kernels
 * and results as moe_grouped_ffn_fp8 (bit for bit), with the workspace taken from a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends (its address is looked up on a device's first call).
 * Calls on one GPU share that array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give unspecified results; calls in one stream's order
 * are safe. Nothing in the array needs to start cleared.
 * Errors: as moe_grouped_ffn_fp8, and MOE_ERR_SCRATCH when
 * moe_grouped_ffn_workspace_bytes(cfg, n_experts, n_rows) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (at the V3 shape, H = 7168 and I = 2048 with 257 experts,
 * up to about 14,000 rows fit; a decode step of 128 tokens has 1,152).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_grouped_ffn_fp8_noalloc(const moe_config* cfg, int32_t n_experts, int64_t n_rows,
                                       int64_t n_tokens, const uint8_t* xq, const float* xs,
                                       const int32_t* row_token, const int32_t* offsets,
                                       const uint8_t* w1, const float* w1s, const uint8_t* w3,
                                       const float* w3s, const uint8_t* w2, const float* w2s,
                                       void* y, moe_dtype yt, void* stream);

/*
 * moe_combine — weighted combine ([digest] section 3.2: y = sum_j gate[j] *
 * ffn_expert[idx[j]](h)) plus the shared experts with gate 1 ([guide] section 3
 * num_shared_experts). FP32 accumulation in fixed order (shared experts 0..N_s-1,
 * then slots 0..k-1), rounded once to bf16.
 *   y_rows    [T*k, H] of dtype yt (rows past T*k, if any, are not read)
 *   row_of    [T, k] int32 (entries < 0 are skipped)
 *   topk_gate [T, k] float
 *   y_shared  [N_s, T, H] of dtype yt, or NULL when N_s == 0 (after moe_permute and one
 *             grouped FFN call over N_r + N_s experts this is y_rows + T*k rows)
 *   out       [T, H] bf16 bits, output
 * Errors: NULL pointers; invalid config; T < 0.
 */
moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, moe_dtype yt,
                       const int32_t* row_of, const float* topk_gate, const void* y_shared,
                       uint16_t* out, void* stream);

/*
 * moe_update_bias — sign-based bias update ([digest] section 3.2 pseudocode: after a
 * step, experts above the mean load T*k/N_r lose gamma, those below gain gamma;
 * section 5.2: statistics over the whole batch). Dead band 0: the comparison is the
 * integer T*k vs N_r*counts[e]; equal load leaves b unchanged. One FP32 rounding.
 *   counts [N_r] int32 (from moe_route over the same T tokens); bias [N_r] float, in/out
 * Errors: NULL pointers; invalid config; T < 0.
 */
moe_status moe_update_bias(const moe_config* cfg, int64_t T, const int32_t* counts,
                           float* bias, void* stream);

/*
 * moe_seq_balance — per-sequence balance statistics of one routing step ([digest]
 * section 3.3: the complementary sequence-level balance loss, alpha times the sum over
 * experts of the expert's share of the sequence's assignments times its mean affinity;
 * section 5.5: the per-sequence allocation entropy as the signal for that loss). The T
 * tokens form T / seq_len sequences of seq_len consecutive tokens. For sequence q:
 *   f_i = (entries of topk_idx in q equal to i) / (top_k * seq_len)
 *   P_i = mean over q's tokens of scores[t, i]
 *   loss[q] = alpha * sum_i f_i * P_i,   entropy[q] = -sum_{f_i > 0} f_i * ln f_i
 * Sums in FP64 in a fixed order (deterministic), each output rounded once to FP32.
 * Entries of topk_idx outside [0, N_r) count for no expert (f no longer sums to 1).
 *   scores    [T, N_r] float (the sigmoid affinities moe_route writes)
 *   topk_idx  [T, top_k] int32
 *   alpha     loss coefficient ([guide] aux_loss_alpha, 0.001)
 *   loss      [T / seq_len] float, output
 *   entropy   [T / seq_len] float, output; NULL skips it
 *   ws        moe_seq_balance_workspace_bytes(cfg, T, seq_len) bytes, 8-byte aligned
 * Errors: NULL pointers (T > 0); invalid config; T < 0, T >= 2^31, seq_len <= 0 or
 * T % seq_len != 0, or more than 2^24 workgroups (SHAPE); workspace NULL or small
 * (WORKSPACE); misaligned workspace (UNSUPPORTED). T == 0 launches nothing.
 */
size_t moe_seq_balance_workspace_bytes(const moe_config* cfg, int64_t T, int64_t seq_len);
moe_status moe_seq_balance(const moe_config* cfg, int64_t T, int64_t seq_len,
                           const float* scores, const int32_t* topk_idx, float alpha,
                           float* loss, float* entropy, void* ws, size_t ws_bytes,
                           void* stream);

/* ===================================================================================
 * Backward pass ([guide] section 3: gemm_dgrad and gemm_wgrad run in FP8 e4m3 like
 * gemm_fprop, moe_gating stays in BF16/FP32; [zhihu] training part: E4M3 in both
 * directions, 1x128 / 128x128 groups, partial-sum promotion, SwiGLU recomputed).
 * Quantisers are straight-through. Each FP8 GEMM quantises its operands along its own
 * contraction axis: 1x128 tiles along H or I for dgrad, and 1x128 tiles along the token
 * axis for wgrad (128 consecutive rows of one expert's segment per tile, from the
 * segment's first row; the last tile may be shorter). Weights keep their 128x128 blocks.
 * Scale rule everywhere: s = fl32(amax / 448) (1 for a zero group), codes =
 * E4M3(fl32(v / s)). Call order for one layer: moe_combine_backward,
 * moe_grouped_ffn_fp8_backward, moe_route_backward, moe_unpermute_sum.
 * =================================================================================== */

/*
 * moe_combine_backward — gradient of the combine ([digest] section 3.2: out_t = shared
 * rows + sum_j gate_tj y_{row_of[t,j]}).
 *   dout      [T, H] bf16 bits: gradient of the layer output
 *   y_rows    [T*(k+N_s), H] (yt = MOE_BF16 or MOE_F32): the forward's expert output rows
 *   row_of, topk_gate: from the forward ([T, k] int32 / float)
 *   row_gate  [T*(k+N_s)] float, output: the gate of every permuted row, gate_tj on row
 *             row_of[t, j] and 1 on the shared rows T*k + s*T + t; rows that no (token,
 *             slot) names are not written. The rows' upstream gradient is
 *             dy_r = row_gate[r] * dout_{token(r)} (one FP32 rounding); it is never stored:
 *             moe_grouped_ffn_fp8_backward forms it from dout and row_gate where it
 *             quantises it.
 *   dgate     [T, k] float, output: sum_h dout_t[h] * y_row[h] (FP32, fixed order); 0 for a
 *             slot with row -1
 * Errors: NULL pointers (T > 0); invalid config; T < 0 or T >= 2^31; yt not BF16/F32.
 */
moe_status moe_combine_backward(const moe_config* cfg, int64_t T, const uint16_t* dout,
                                const void* y_rows, moe_dtype yt, const int32_t* row_of,
                                const float* topk_gate, float* row_gate, float* dgate,
                                void* stream);

/*
 * moe_route_backward — gradient of the gates through the router, in FP32 ([digest]
 * section 3.2: gate_j = rho * s_j / sum of the selected s, s = sigmoid(x . W_r^T); the
 * bias and the group limit only select, so the selection carries no gradient).
 *   ds_m = (rho / Z) (dgate_m - sum_j dgate_j gate_j / rho) for the selected m, Z = sum of
 *   the selected s; dlogit = ds * s * (1 - s); dx = dlogit . W_r; dW_r[e] = sum over the
 *   rows of e's segment (row order) of dlogit * x_token.
 *   x [T, H] (xt), w_router [N_r, H] float (plain row-major), scores [T, N_r] (moe_route's
 *   s), topk_idx [T, k], dgate [T, k], offsets / row_token / row_of from moe_permute.
 *   dx        [T, H] float, output (the router's share of the input gradient)
 *   dw_router [N_r, H] float, output
 *   ws        moe_route_backward_workspace_bytes(cfg, T) bytes
 * Errors: NULL pointers (T > 0; offsets and dw_router always); invalid config; T out of
 * range (SHAPE); xt not BF16/F32 (DTYPE); workspace missing or small (WORKSPACE).
 */
size_t moe_route_backward_workspace_bytes(const moe_config* cfg, int64_t T);
moe_status moe_route_backward(const moe_config* cfg, int64_t T, const void* x, moe_dtype xt,
                              const float* w_router, const float* scores,
                              const int32_t* topk_idx, const float* dgate,
                              const int32_t* offsets, const int32_t* row_token,
                              const int32_t* row_of, float* dx, float* dw_router, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * moe_unpermute_sum — input gradient per token from its permuted rows ([digest] section
 * 3.2: each token's output sums its experts, so its input gradient sums theirs):
 * out_t = bf16( sum_s rows[T*k + s*T + t] + sum_j rows[row_of[t, j]] + extra_t ), FP32 in
 * that order. rows [T*(k+N_s), H] (rt = BF16/F32); extra [T, H] float or NULL; out [T, H]
 * bf16 bits. Errors: NULL pointers (T > 0); invalid config; T out of range; bad rt.
 */
moe_status moe_unpermute_sum(const moe_config* cfg, int64_t T, const void* rows, moe_dtype rt,
                             const int32_t* row_of, const float* extra, uint16_t* out,
                             void* stream);

/*
 * moe_transpose_fp8_blocks — set-up for the dgrad GEMMs, which contract the weights over
 * their other axis: dst[e][c][col0 + r] = src[e][r][c] for E4M3 codes ([E, R, C] ->
 * rows of dst_cols), and each 128x128 block scale moves with its block:
 * dst_scales[e][c/128][(col0 + r)/128] = src_scales[e][r/128][c/128]. The result is
 * row-major codes for moe_pack_fp8_weights (W2^T: [E, I, H]; [W1^T | W3^T]: [E, H, 2I]
 * from two calls with col0 = 0 and I).
 * Errors: R, C, dst_cols, col0 not multiples of 128, col0 + R > dst_cols, E > 65535
 * (SHAPE); NULL pointers.
 */
moe_status moe_transpose_fp8_blocks(int64_t E, int64_t R, int64_t C, const uint8_t* src,
                                    const float* src_scales, uint8_t* dst, float* dst_scales,
                                    int64_t dst_cols, int64_t col0, void* stream);

/*
 * moe_grouped_ffn_fp8_backward — backward of the grouped SwiGLU experts with FP8 GEMMs, on
 * the same permuted rows and segments as moe_grouped_ffn_fp8 (routed then shared).
 *   SwiGLU inputs: a = xq W1^T, b = xq W3^T as the training forward kept them
 *              (a_saved, b_saved from moe_grouped_ffn_fp8_gate_up_train), or, when both
 *              are NULL, recomputed by the FP8 fprop GEMMs on the forward's codes (the
 *              same launch, so the same values bit for bit).
 *   dgrad:     dh = dy W2 with dy_r = fl32(row_gate[r] * dout[row_token[r]]) (dy in 1x128
 *              tiles along H); dg = dh b silu'(a), du = dh silu(a)
 *              (FP32); dx_rows = dg W1 + du W3 ([dg | du] in 1x128 tiles along I, one
 *              GEMM over K = 2I with the packed [W1^T | W3^T]).
 *   wgrad:     dW2 = dy^T h, dW1 = dg^T x, dW3 = du^T x with h = silu(a) b (FP32) and x
 *              the layer input rows; every operand in 128-row tiles along the token axis.
 *   Rows with row_token < 0 count as zero rows (their dy is ignored).
 *   xq, xs       [T, H] u8 / [T, H/128] float: the forward's activation codes and scales
 *                (read only to recompute a and b; may be NULL with a_saved, b_saved)
 *   x            [T, H] (xt = BF16/F32): the layer input, 16-byte aligned
 *   w1, w3 (+s)  the forward's packed weights; w2t (+s): packed W2^T [E, I, H] with
 *                scales [E, I/128, H/128]; w13t (+s): packed [W1^T | W3^T] [E, H, 2I]
 *                with scales [E, H/128, 2I/128] (moe_transpose_fp8_blocks, then
 *                moe_pack_fp8_weights)
 *   a_saved, b_saved  [n_rows, I] float each or both NULL: the forward's SwiGLU inputs
 *   dout         [T, H] bf16 bits, 16-byte aligned: the layer's upstream gradient (rows of dy
 *                are gated copies)
 *   row_gate     [n_rows] float (moe_combine_backward) or NULL (every row's gate 1)
 *   dx_rows      [n_rows, H] output (dxt = BF16/F32)
 *   dw1, dw3     [E, I, H] and dw2 [E, H, I] outputs (dwt = BF16/F32): FP32-promoted
 *                sums, written for every expert (zero for an expert without rows)
 *   ws           moe_grouped_ffn_backward_workspace_bytes(cfg, E, n_rows) bytes
 * Errors: NULL pointers (one of a_saved, b_saved NULL and the other not is NULL too);
 * invalid config; scale_mode != 0 (UNSUPPORTED); E outside 1..1024, n_rows or T out of
 * range (SHAPE); bad dtypes (DTYPE); workspace (WORKSPACE);
 * n_rows * H or n_rows * 2I >= 2^32, H or 2I > 16384, or max(H, I) * (n_rows + 128 E)
 * >= 2^31 (the token-axis operands' 32-bit offsets; about 266,000 rows at the V3 shape),
 * or x or dout not 16-byte aligned (UNSUPPORTED).
 */
size_t moe_grouped_ffn_backward_workspace_bytes(const moe_config* cfg, int32_t n_experts,
                                                int64_t n_rows);
moe_status moe_grouped_ffn_fp8_backward(
    const moe_config* cfg, int32_t n_experts, int64_t n_rows, int64_t n_tokens, const uint8_t* xq,
    const float* xs, const void* x, moe_dtype xt, const int32_t* row_token, const int32_t* offsets,
    const uint8_t* w1, const float* w1s, const uint8_t* w3, const float* w3s, const uint8_t* w2t,
    const float* w2ts, const uint8_t* w13t, const float* w13ts, const float* a_saved,
    const float* b_saved, const uint16_t* dout, const float* row_gate, void* dx_rows,
    moe_dtype dxt, void* dw1, void* dw3, void* dw2, moe_dtype dwt, void* ws, size_t ws_bytes,
    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
