// Chunk staging shared by the two attention kernels.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: the 512-d latent of a
// row is both its key and its value; section 2.4.4: main KV rows are E2M1
// codes with one E4M3 scale per 16 channels, SWA rows are E4M3 with one fp32
// scale per row.
//
// The rows of one 64-row chunk are dequantised once to fp16 and written
// row-major to LDS.  The row stride KV_LD is 536 halves = 268 words, 12 banks
// apart modulo the 64 banks: the 16 rows of a QK^T operand read (16 bytes
// per lane) land on 16 disjoint 4-bank groups, the 4 rows x 4 column groups
// of a transposing PV read (8 bytes per lane) on 16 disjoint 2-bank pairs,
// and the 16 rows of a staging write on 16 disjoint groups.  (A stride 8
// banks apart put rows r and r + 8 of a QK^T read on the same banks.)
//   main rows  E2M1 x E4M3 products are exact in fp16 (at most 6 significant
//              bits, magnitudes in [2^-10, 2688]); they serve as K and V.
//   SWA rows   the E4M3 values unscaled (exact) serve as K, the row scale
//              being applied to the scores; a second copy scaled by the row
//              scale (rounded once to fp16) serves as V.
// QK^T reads a K row as the B operand (8 consecutive dims per lane); PV
// reads 8 consecutive rows of one dim as its B operand with two gfx950
// transposing LDS reads (ds_read_b64_tr_b16), so no transposed copy of V
// is ever written.
#pragma once

#include "common.h"
#include "launch.h"

namespace csa2 {

// e^x on the hardware exponential, 2^(x log2 e) by v_exp_f32.  Rounding
// x log2 e adds at most |x| 2^-24 relative error, far below the fp16
// rounding the softmax weights get before the P V product; e^-inf = 0.
__device__ __forceinline__ float exp_hw(float x) { return __expf(x); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

constexpr int CH_ROWS = 64;             // rows per chunk
constexpr int KV_LD = D_LAT + 24;       // fp16 row stride of a staged chunk

// One thread's share of a chunk row: NT threads cover 64 rows, NT / 64
// threads per row, DIMS consecutive dims each.
template <int NT>
struct RawShare {
  static constexpr int PARTS = NT / CH_ROWS;
  static constexpr int DIMS = D_LAT / PARTS;          // 128 (256 threads) or 64 (512)
  static constexpr int MW = DIMS / 32;                // 16-byte words of E2M1 codes
  static constexpr int SW = DIMS / 16;                // 16-byte words of E4M3 SWA bytes
  u32x4_t c[SW];
  uint64_t s;                                         // DIMS / 16 E4M3 scale bytes (main)
};

// Issue the loads of one share: main-KV entry `off` (flat entry index) or
// SWA row `off` (flat row index); `off` must address a readable row.
template <int NT>
__device__ __forceinline__ void load_share(RawShare<NT>& r, bool is_main, int64_t off, int part,
                                           const uint8_t* __restrict__ kv_codes,
                                           const uint8_t* __restrict__ kv_scales,
                                           const uint8_t* __restrict__ swa_codes) {
  using R = RawShare<NT>;
  const uint8_t* base = is_main ? kv_codes + off * (D_LAT / 2) + part * (R::DIMS / 2)
                                : swa_codes + off * D_LAT + part * R::DIMS;
#pragma unroll
  for (int i = 0; i < R::MW; ++i) r.c[i] = ((const u32x4_t*)base)[i];
  if (is_main) {
    const uint8_t* sp = kv_scales + off * (D_LAT / 16) + part * (R::DIMS / 16);
    r.s = R::DIMS / 16 == 8 ? *(const uint64_t*)sp : (uint64_t)*(const uint32_t*)sp;
  } else {
#pragma unroll
    for (int i = R::MW; i < R::SW; ++i) r.c[i] = ((const u32x4_t*)base)[i];
  }
}

// Eight E2M1 codes of a word times an fp16 scale pair: converted at scale 1,
// then one packed fp16 multiply per pair (exact, see above).
__device__ __forceinline__ f16x8_t fp4x8_f16(uint32_t w, f16x2_t s2) {
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight E4M3FN bytes (two words) to fp16 at scale 1 (exact).
__device__ __forceinline__ f16x8_t fp8x8_f16(uint32_t lo, uint32_t hi) {
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Dequantise one share into row `row` of kv (and, for SWA rows with
// V_COPY, the copy scaled by the row scale into kv2; without it the caller
// applies the row scale to P instead).  An invalid main row is written as
// zeros and an invalid SWA row gets a zero V (copy): the caller masks their
// scores, and zero values keep P V finite whatever bytes the row held.
template <int NT, bool V_COPY = true>
__device__ __forceinline__ void store_share(const RawShare<NT>& r, bool is_main, bool valid,
                                            float sig, _Float16* __restrict__ kv,
                                            _Float16* __restrict__ kv2, int row, int part) {
  using R = RawShare<NT>;
  _Float16* dst = kv + row * KV_LD + part * R::DIMS;
  if (is_main) {
    const uint32_t sb_lo = valid ? (uint32_t)r.s : 0u;
    const uint32_t sb_hi = valid ? (uint32_t)(r.s >> 32) : 0u;
#pragma unroll
    for (int p = 0; p < R::DIMS / 32; ++p) {          // scale groups 2p, 2p+1 (16 dims each)
      const uint32_t sw = p < 2 ? sb_lo : sb_hi;
      const f16x2_t sp = (p & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * p + h;
        const f16x2_t s2 = {sp[h], sp[h]};
        const uint32_t w0 = r.c[(2 * g) >> 2][(2 * g) & 3];
        const uint32_t w1 = r.c[(2 * g + 1) >> 2][(2 * g + 1) & 3];
        *(f16x8_t*)(dst + 16 * g) = fp4x8_f16(w0, s2);
        *(f16x8_t*)(dst + 16 * g + 8) = fp4x8_f16(w1, s2);
      }
    }
  } else if (!V_COPY) {
    const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;   // code 0 is +0
#pragma unroll
    for (int i = 0; i < R::SW; ++i) {                 // 16 dims per word
      *(f16x8_t*)(dst + 16 * i) = fp8x8_f16(r.c[i][0] & keep, r.c[i][1] & keep);
      *(f16x8_t*)(dst + 16 * i + 8) = fp8x8_f16(r.c[i][2] & keep, r.c[i][3] & keep);
    }
  } else {
    _Float16* dst2 = kv2 + row * KV_LD + part * R::DIMS;
    const float g = valid ? sig : 0.f;
#pragma unroll
    for (int i = 0; i < R::SW; ++i) {                 // 16 dims per word
      *(f16x8_t*)(dst + 16 * i) = fp8x8_f16(r.c[i][0], r.c[i][1]);
      *(f16x8_t*)(dst + 16 * i + 8) = fp8x8_f16(r.c[i][2], r.c[i][3]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f16x8_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = r.c[i][2 * hh + (q >> 1)];
          const f32x2_t f = (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                                    : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
          v[2 * q] = (_Float16)(f[0] * g);
          v[2 * q + 1] = (_Float16)(f[1] * g);
        }
        *(f16x8_t*)(dst2 + 16 * i + 8 * hh) = v;
      }
    }
  }
}

// B operand of S = Q K^T for k-step s: row `row` of the staged chunk,
// dims 32 s + 8 qd .. +7.
__device__ __forceinline__ f16x8_t qk_b(const _Float16* kv, int row, int s, int qd) {
  return *(const f16x8_t*)(kv + row * KV_LD + 32 * s + 8 * qd);
}

// B operand of O += P V for 16x16x32: lane l gets rows kbase + 8 (l / 16)
// .. +7 of dim n0 + l % 16.  In each 16-lane group the transposing read
// gives lane j element e = the element (j & 3) of the 4 that lane 4 e +
// (j >> 2) addressed; lane i therefore addresses row kbase' + (i >> 2),
// dims n0 + 4 (i & 3) .. +3.
__device__ __forceinline__ f16x8_t pv_b(const _Float16* v, int kbase, int n0, int lane) {
  const int i = lane & 15;
  const _Float16* p = v + (kbase + 8 * (lane >> 4) + (i >> 2)) * KV_LD + n0 + 4 * (i & 3);
  typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 4 * KV_LD));
  const f16x4_t a = __builtin_bit_cast(f16x4_t, lo), b = __builtin_bit_cast(f16x4_t, hi);
  return f16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// fp16 query factor of a head whose largest |q| is `mx`: 2^e with mx 2^e in
// [2^13, 2^14), so every component above 2^-24 of the head's largest
// converts to fp16 exactly and none overflows.
__device__ __forceinline__ int q_exponent(float mx) {
  if (!(mx > 0.f) || !(mx < INFINITY)) return 0;
  int e = 13 - ilogbf(mx);
  return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// Rotary position embedding around the attention (RopeArgs, launch.h).  The
// rotated channels are at most the last 64 (the width of the query steps 14
// and 15, which carry a second, low fp16 term of the rotated query so that
// the logits keep fp32 accuracy).
constexpr int ROPE_MAX_DIMS = 64;
constexpr int ROPE_MAX_PAIRS = ROPE_MAX_DIMS / 2;

static_assert(ROPE_MAX_PAIRS <= 32, "RopeArgs::freq holds 32 pairs");

// cos and sin of pair i's angle at position pos: the angle pos * freq[i] is
// formed and reduced modulo 2 pi in fp64 (it reaches 10^6 radians at 1M
// positions), then its cos and sin are taken in fp32.
__device__ inline f32x2_t rope_cs(int64_t pos, int i, const RopeArgs& rp) {
  const double two_pi = 6.283185307179586476925;
  double ang = (double)pos * rp.freq[i];
  ang -= two_pi * rint(ang * (1.0 / two_pi));
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  return f32x2_t{cs, sn};
}

// The table of one query's (cos, sin) per pair, filled by the workgroup's
// NT threads (with a barrier) when there is a rotation.
template <int NT>
__device__ __forceinline__ void rope_table(const RopeArgs& rp, int q, f32x2_t* tab) {
  if (rp.dims > 0) {                                  // uniform: a kernel argument
    const int64_t pos = rp.q_pos[q];
    for (int i = threadIdx.x; i < rp.dims / 2; i += NT) tab[i] = rope_cs(pos, i, rp);
    __syncthreads();
  }
}

// Turn the pair (x[0], x[1]) = channels (d, d + 1), d even, by the table's
// angle (sign +1) or its opposite (sign -1), if d is a RoPE channel.
__device__ __forceinline__ void rope_pair(float& a, float& b, int d, int dims, const f32x2_t* tab,
                                          float sign) {
  const int base = D_LAT - dims;
  if (dims > 0 && d >= base) {
    const f32x2_t cs = tab[(d - base) >> 1];
    const float sn = sign * cs[1];
    const float na = a * cs[0] - b * sn, nb = a * sn + b * cs[0];
    a = na;
    b = nb;
  }
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One output value of channel d held by this lane, whose pair partner
// (channel d ^ 1) the neighbouring lane (lane ^ 1) holds: turned back by
// the query's angle when d is a RoPE channel.  Every lane of the wave must
// call it (it exchanges values).
__device__ __forceinline__ float rope_out_lane(float v, int d, int dims, const f32x2_t* tab) {
  const float w = __shfl_xor(v, 1);
  const int base = D_LAT - dims;
  if (dims > 0 && d >= base) {
    const f32x2_t cs = tab[(d - base) >> 1];
    // inverse turn: (a, b) -> (a cos + b sin, b cos - a sin)
    v = (d & 1) ? v * cs[0] - w * cs[1] : v * cs[0] + w * cs[1];
  }
  return v;
}

}  // namespace csa2
