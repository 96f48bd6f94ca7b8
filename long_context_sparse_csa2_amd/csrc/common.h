// Device helpers shared by the CSA2 kernels: number formats, MFMA wrappers,
// order-preserving score keys.  gfx950 (CDNA4) only.
//
// Formats (report digest "DeepSeek-V4.1-Flash", section 2.4.4; bit layouts
// from the OCP MX v1.0 and OCP FP8 specifications):
//   E2M1    s|e1e0|m, bias 1: {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign
//   E4M3FN  s|eeee|mmm, bias 7, max 448, S.1111.111 = NaN
//   E8M0    2^(e - 127)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace csa2 {

constexpr int D_LAT = 512;
constexpr int H_IDX = 32;
constexpr int D_IDX = 128;
constexpr int H_ATT = 64;

// ------------------------------------------------------------- decoders
// |E2M1| for a 3-bit magnitude code, built from its bit fields.
__device__ __forceinline__ float e2m1_mag(uint32_t n) {
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  return e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
}

__device__ __forceinline__ float e2m1_val(uint32_t n) {
  const float v = e2m1_mag(n & 7u);
  return (n & 8u) ? -v : v;
}

__device__ __forceinline__ float e4m3_val(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  return (c & 0x80u) ? -v : v;
}

// 2^(c - 127) for an E8M0 byte (0xFF, NaN in the format, is not produced).
__device__ __forceinline__ float e8m0_val(uint32_t c) {
  return c == 0 ? 0x1p-127f : __uint_as_float(c << 23);
}

// ------------------------------------------------------------- encoders
// RNE to E4M3FN of a non-negative value, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0x1p-6f) return (uint32_t)rintf(v * 512.0f);        // subnormal step 2^-9
  int ex;
  (void)frexpf(v, &ex);                                          // v = f 2^ex, f in [0.5, 1)
  const int e = ex - 1;
  const float q = rintf((ldexpf(v, -e) - 1.0f) * 8.0f);         // exact scaling, RNE
  const uint32_t code = ((uint32_t)(e + 7) << 3) + (uint32_t)q;  // q == 8 carries into e
  return code > 0x7Eu ? 0x7Eu : code;
}

// RNE of x / s to E2M1 with saturation at 6, evaluated as comparisons of |x|
// with the exact midpoints t * s (t has at most 3 significant bits and s at
// most 4, so every product is exact in fp32).  A tie goes to the even code:
// the midpoints 0.75, 1.75, 3.5 round up, 0.25, 1.25, 2.5, 5 round down.
// The sign bit is set iff x < 0.
__device__ __forceinline__ uint32_t e2m1_encode(float x, float s) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) +
                     (uint32_t)(a > 1.25f * s) + (uint32_t)(a >= 1.75f * s) +
                     (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
                     (uint32_t)(a > 5.0f * s);
  return c | (x < 0.0f ? 8u : 0u);
}

// ------------------------------------------------------------ conversions
__device__ __forceinline__ uint16_t bf16_bits_exact(float v) {   // v exactly representable
  return (uint16_t)(__float_as_uint(v) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Eight E2M1 codes of a 32-bit word (low nibble = first element) times a
// power-of-two scale (an E8M0 value), to bf16, with the gfx950 scaled FP4
// conversion (two elements per call, byte_sel picks the byte).  The
// instruction applies only the exponent of its fp32 scale operand, so it is
// exact for power-of-two scales and must not be given any other scale.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16_pow2(uint32_t w, float scale_pow2) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_pow2, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_pow2, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_pow2, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_pow2, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight E2M1 codes times an arbitrary fp32 scale (an E4M3 value), to bf16:
// converted to fp32 at scale 1, multiplied in fp32 and truncated to bf16,
// which is exact because every product has at most 6 significant bits.
__device__ __forceinline__ uint32_t bf16_pair_exact(f32x2_t f, float scale) {
  const uint32_t lo = __float_as_uint(f[0] * scale), hi = __float_as_uint(f[1] * scale);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);         // upper halves: {lo, hi}
}

__device__ __forceinline__ bf16x8_t fp4x8_to_bf16_scaled(uint32_t w, float scale) {
  uint32_t packed[4];
  packed[0] = bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), scale);
  packed[1] = bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), scale);
  packed[2] = bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), scale);
  packed[3] = bf16_pair_exact(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), scale);
  return __builtin_bit_cast(bf16x8_t, packed);
}

// Eight E2M1 codes times an E4M3 scale, to fp16: converted at scale 1, then
// one packed fp16 multiply per pair (exact: E4M3 values and the products
// are fp16 numbers).
__device__ __forceinline__ f16x8_t fp4x8_to_f16_scaled(uint32_t w, float scale) {
  const _Float16 sh = (_Float16)scale;
  const f16x2_t s2 = {sh, sh};
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The same conversion written out with integer/bit operations (used by the
// device self-test to check the hardware instruction).
__device__ __forceinline__ float fp4_scaled_soft(uint32_t w, int i, float scale) {
  return e2m1_val((w >> (4 * i)) & 15u) * scale;
}

// Eight E4M3FN bytes (two words, byte 0 first) to bf16 with the gfx950 FP8
// conversion at scale 1 (exact: every E4M3FN value is a bf16 value).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight E4M3FN bytes times an fp32 scale to fp16: decoded to fp32 at scale
// 1 (exact), multiplied in fp32, rounded once to fp16.
__device__ __forceinline__ f16x8_t fp8x8_to_f16_scaled(uint32_t lo, uint32_t hi, float scale) {
  const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false);
  const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, true);
  const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false);
  const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true);
  f16x8_t r;
  r[0] = (_Float16)(p0[0] * scale); r[1] = (_Float16)(p0[1] * scale);
  r[2] = (_Float16)(p1[0] * scale); r[3] = (_Float16)(p1[1] * scale);
  r[4] = (_Float16)(p2[0] * scale); r[5] = (_Float16)(p2[1] * scale);
  r[6] = (_Float16)(p3[0] * scale); r[7] = (_Float16)(p3[1] * scale);
  return r;
}

// max(x, 0) as one integer max on the bit pattern: every float with the
// sign bit set (including -0) becomes +0, the rest is unchanged.
__device__ __forceinline__ float relu_f32(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ------------------------------------------------------------------ MFMA
// 32x32x16 bf16: A lane l holds A[l%32][8(l/32) .. +7]; B lane l holds
// B[8(l/32) .. +7][l%32]; D lane l element j is D[8(j/4) + 4(l/32) + j%4][l%32].
__device__ __forceinline__ f32x16_t mfma32_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32: A lane l holds A[l%16][8(l/16) .. +7]; B lane l holds
// B[8(l/16) .. +7][l%16]; D lane l element j is D[4(l/16) + j][l%16].
__device__ __forceinline__ f32x4_t mfma16_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------- lane-pair sums / maxima
// x combined with the value of lane l ^ 16 (or l ^ 32), by the gfx950
// row-swapping permutes (VALU, no LDS round trip); both lanes of a pair get
// the same result, bit for bit, since max and a two-term sum do not depend
// on the operand order.  Every lane must be active.
__device__ __forceinline__ float lanes_max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lanes_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lanes_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lanes_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t lanes_max16u(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}

// ------------------------------------------------------------ wave scans
// Inclusive scan over the 64 lanes of a wave with DPP: Hillis-Steele shifts
// inside each 16-lane row, then the row_bcast:15 / row_bcast:31 steps carry
// the row totals across rows.  `ident` is the identity of `op`.  Must be
// called with every lane active.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, Op op, uint32_t ident) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) { return wave_scan_dpp(v, OpAdd(), 0u); }
__device__ __forceinline__ uint32_t wave_max_all(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(v, OpMax(), 0u), 63);
}
__device__ __forceinline__ uint32_t wave_min_all(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(v, OpMin(), 0xFFFFFFFFu), 63);
}

// Max / sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), every
// lane getting the result: xor-1 and xor-2 quad permutations, then the
// half-row and row mirrors (each step pairs groups that already agree, so
// all 16 lanes end with the same value).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_movu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xb1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4e>(v));     // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));    // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));    // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xb1>(v);
  v += dpp_mov<0x4e>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// ------------------------------------------------------------ score keys
// Order-preserving map of fp32 to uint32 (larger value -> larger key);
// -0 is folded onto +0 so that equal values give equal keys.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Number of levels of 8-way maxima above the scores and their sizes.
constexpr int SEL_CAP = 16384;      // candidates one selection workgroup holds
constexpr int SEL_MAX_LEVELS = 4;   // 8^4 * SEL_CAP covers 2^26 columns

__host__ __device__ inline int64_t groups_at(int64_t n, int lvl) {
  int64_t g = n;
  for (int i = 0; i < lvl; ++i) g = (g + 7) / 8;
  return g;
}

}  // namespace csa2
