// Internal interface of the grouped FP8 GEMM kernel (ffn.hip) for the backward pass:
// a tile plan over expert segments and the phase-2 kernel as a plain grouped GEMM.
#pragma once

#include "common.h"

namespace moe {

// Bytes of a tile plan for n_rows permuted rows over n_experts segments.
size_t ffn_plan_bytes(int32_t n_experts, int64_t n_rows);

// Plan tiles of the segments offsets[0..n_experts] into `plan` (ffn_plan_bytes bytes).
moe_status ffn_plan_launch(const int32_t* offsets, int32_t n_experts, int64_t n_rows, void* plan,
                           hipStream_t s);

// y[rows, N] = A[rows, K] x W_e[N, K]^T for every planned tile (expert e's segment):
// A = aq (E4M3, row-major, stride K) with 1x128 scales as_cm chunk-major [K/128][n_rows];
// W packed as moe_pack_fp8_weights lays [E][N][K], block scales wsc [E][N/128][K/128].
// FP32 promotion per 128-wide K chunk; y is bf16 or f32, row-major, stride N.
moe_status ffn_grouped_gemm_launch(const void* plan, int32_t n_experts, int64_t n_rows,
                                   const uint8_t* aq, const float* as_cm, const uint8_t* w,
                                   const float* wsc, int N, int K, void* y, moe_dtype yt,
                                   hipStream_t s);

// The gate/up GEMMs of the forward with their FP32 results kept: a = x W1^T and
// b = x W3^T ([n_rows, I] each) for every planned tile, x gathered from xq by row_token
// (rows without a token give zeros). xsp: scratch for the gathered scales, chunk-major
// [H/128][n_rows].
moe_status ffn_recompute_launch(const void* plan, int32_t n_experts, int64_t n_rows,
                                int64_t n_tokens, const uint8_t* xq, const float* xs,
                                const int32_t* row_token, const uint8_t* w1, const float* w1s,
                                const uint8_t* w3, const float* w3s, int H, int I, float* xsp,
                                float* a_out, float* b_out, hipStream_t s);

}  // namespace moe
