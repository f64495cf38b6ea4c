// Shared helpers of the gfx950 MoE library: status plumbing, config validation,
// E4M3 encoding, bf16 conversion and wavefront reductions. gfx950 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_fp8.h"

#define MOE_TRY_HIP(expr)                         \
  do {                                            \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

namespace moe {

constexpr int kWave = 64;
constexpr int kTile = 128;            // 1x128 activation tiles, 128x128 weight blocks
constexpr float kE4M3Max = 448.0f;
constexpr int kMaxRouted = 512;
constexpr int kMaxShared = 16;
constexpr int kMaxTopK = 16;
constexpr int kMaxGroups = 64;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Host-side validation of a layer configuration (the ranges stated in moe_fp8.h).
inline moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_NULL;
  if (c->hidden <= 0 || c->hidden % kTile) return MOE_ERR_SHAPE;
  if (c->inter <= 0 || c->inter % kTile) return MOE_ERR_SHAPE;
  if (c->n_routed < 1 || c->n_routed > kMaxRouted) return MOE_ERR_SHAPE;
  if (c->n_shared < 0 || c->n_shared > kMaxShared) return MOE_ERR_SHAPE;
  if (c->scale_mode != 0 && c->scale_mode != 1) return MOE_ERR_UNSUPPORTED;
  if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->n_routed) return MOE_ERR_SHAPE;
  if (c->n_group < 1 || c->n_group > kMaxGroups || c->n_routed % c->n_group) return MOE_ERR_SHAPE;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_SHAPE;
  const int gsz = c->n_routed / c->n_group;
  if (c->group_topn < 1 || c->group_topn > gsz) return MOE_ERR_SHAPE;
  if ((int64_t)c->topk_group * gsz < c->top_k) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// ---------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------

// OCP E4M3FN encoding of a float32 value: nearest finite value, ties to even mantissa,
// saturating at +-448, sign kept (-0 -> 0x80), NaN -> 0x7F | sign. gfx950's
// v_cvt_pk_fp8_f32 rounds to nearest even on this grid (subnormals included) but turns
// magnitudes from 464 up into NaN, hence the clamp to +-448 first; NaN takes its own path
// because the clamp would turn it into a number.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float c = fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFFu;
  return v == v ? code : (((__float_as_uint(v) >> 24) & 0x80u) | 0x7Fu);
}

// Four values encoded as by e4m3_encode, packed little-endian (a in the low byte), two
// per conversion instruction.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const auto cl = [](float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  if (!(a == a && b == b && c == c && d == d))
    return e4m3_encode(a) | (e4m3_encode(b) << 8) | (e4m3_encode(c) << 16) | (e4m3_encode(d) << 24);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two float32 values -> packed bf16 (a in the low half), round to nearest even, through
// gfx950's v_cvt_pk_bf16_f32. For outputs; exact splits use f32_to_bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Scale of a quantisation group from its amax: fl32(amax / 448), or 1 when that is 0.
__device__ __forceinline__ float group_scale(float amax) {
  const float s = __fdiv_rn(amax, kE4M3Max);
  return s == 0.0f ? 1.0f : s;
}

// Power-of-two scale of a group: the smallest 2^k with amax / 2^k <= 448, k >= -126; 1 for
// amax == 0. With amax = m * 2^E (m in [1, 2)) and 448 = 1.75 * 2^8, k = E - 8, plus one
// when m > 1.75 (fraction bits above 0x600000).
__device__ __forceinline__ float group_scale_pow2(float amax) {
  if (amax == 0.0f) return 1.0f;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFFu) - 127;
  int k = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  k = max(k, -126);
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// 1 / s for a power-of-two s in [2^-126, 2^126] (exact).
__device__ __forceinline__ float inv_pow2(float s) {
  return __uint_as_float((254u - ((__float_as_uint(s) >> 23) & 0xFFu)) << 23);
}

// E8M0 exponent byte of a power-of-two float (the MFMA block-scale operand: 2^(e - 127)).
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

}  // namespace moe
