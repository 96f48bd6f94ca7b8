// Device self-test of the gfx950 instructions the kernels depend on, each
// checked against plain integer/bit code on the same device:
//   0  FP4 -> bf16 with a power-of-two scale in the conversion (E8M0 path)
//   1  FP4 -> bf16 times each E4M3 scale (main-KV path, fp32 multiply)
//   2  MFMA 32x32x16 bf16 row/column placement of A, B and D
//   3  MFMA 16x16x32 bf16 placement
//   4  MFMA 16x16x32 fp16 placement
//   5  FP4 -> fp16 times each E4M3 scale (packed fp16 multiply)
//   6  DPP wave scan / max / min against a lane loop
//   7  E4M3FN -> bf16 / fp16 (times scales) for all 256 codes but NaN
//   8  fp32 -> E2M1 with a power-of-two scale (the MXFP4 quantisation of
//      the indexer K and query): round to nearest even, saturating at 6,
//      against the compare-based encoder, ties and the extreme scales
// Each counter holds the number of mismatching values (0 = pass).
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int ST_COUNT = 9;

__device__ __forceinline__ int st_a(int m, int k) { return ((m * 7 + k * 3) % 9) - 4; }
__device__ __forceinline__ int st_b(int k, int n) { return ((k * 5 + n * 11) % 7) - 3; }

__global__ __launch_bounds__(64) void k_selftest(int32_t* counts) {
  const int l = threadIdx.x;
  int bad_pow2 = 0, bad_bf = 0, bad_f16 = 0;
  const float pow2[6] = {1.0f, 0.5f, 0x1p-9f, 0x1p-20f, 0x1p20f, 0x1p-126f};
  for (int v = 0; v < 256; ++v) {
    const uint32_t w = (uint32_t)v | ((uint32_t)((v ^ l) & 255) << 8) |
                       ((uint32_t)((v + 3 * l) & 255) << 16) | ((uint32_t)((v * 5 + l) & 255) << 24);
    for (int si = 0; si < 6; ++si) {
      const bf16x8_t hw = fp4x8_to_bf16_pow2(w, pow2[si]);
      for (int i = 0; i < 8; ++i) {
        const float got = (float)hw[i];
        const float want = fp4_scaled_soft(w, i, pow2[si]);
        bad_pow2 += !(got == want && signbit(got) == signbit(want));
      }
    }
    // every positive finite E4M3FN scale; lane l takes codes l, l + 64
    for (int sc = l + 1; sc < 0x7F; sc += 64) {
      const float s = e4m3_val((uint32_t)sc);
      const bf16x8_t hb = fp4x8_to_bf16_scaled(w, s);
      const f16x8_t hh = fp4x8_to_f16_scaled(w, s);
      for (int i = 0; i < 8; ++i) {
        const float want = fp4_scaled_soft(w, i, s);
        const float gb = (float)hb[i], gh = (float)hh[i];
        bad_bf += !(gb == want);
        bad_f16 += !(gh == want);
      }
    }
  }
  {  // DPP wave scans
    const uint32_t x = (uint32_t)((l * 37 + 11) % 101);
    const uint32_t inc = wave_incl_sum(x);
    const uint32_t mxv = wave_max_all(x), mnv = wave_min_all(x + 5);
    uint32_t ref = 0, rmx = 0, rmn = 0xFFFFFFFFu;
    for (int j = 0; j < 64; ++j) {
      const uint32_t y = (uint32_t)((j * 37 + 11) % 101);
      if (j <= l) ref += y;
      rmx = y > rmx ? y : rmx;
      rmn = y + 5 < rmn ? y + 5 : rmn;
    }
    atomicAdd(&counts[6], (int)(inc != ref) + (int)(mxv != rmx) + (int)(mnv != rmn));
  }
  {  // FP8 E4M3FN conversions: lane l checks codes 4l .. 4l+3 in every byte position
    int bad8 = 0;
    const float scales[3] = {1.0f, 0.0137f, 3.5f};
    for (int rot = 0; rot < 4; ++rot) {
      uint32_t lo = 0, hi = 0;
      for (int b = 0; b < 4; ++b) {
        lo |= (uint32_t)((4 * l + ((b + rot) & 3)) & 255) << (8 * b);
        hi |= (uint32_t)((4 * l + ((b + rot + 2) & 3)) & 255) << (8 * b);
      }
      const bf16x8_t vb = fp8x8_to_bf16(lo, hi);
      for (int si = 0; si < 3; ++si) {
        const f16x8_t vh = fp8x8_to_f16_scaled(lo, hi, scales[si]);
        for (int i = 0; i < 8; ++i) {
          const uint32_t c = ((i < 4 ? lo : hi) >> (8 * (i & 3))) & 255u;
          if ((c & 0x7Fu) == 0x7Fu) continue;                   // NaN codes
          const float want = e4m3_val(c);
          if (si == 0) bad8 += !((float)vb[i] == want && signbit((float)vb[i]) == signbit(want));
          bad8 += (float)vh[i] != (float)(_Float16)(want * scales[si]);
        }
      }
    }
    atomicAdd(&counts[7], bad8);
  }
  atomicAdd(&counts[0], bad_pow2);
  atomicAdd(&counts[1], bad_bf);
  atomicAdd(&counts[5], bad_f16);

  {  // fp32 -> E2M1 scaled: magnitudes v / 32 (0 .. 7.97, every tie) times 2^e
    const int exps[7] = {-127, -126, -20, -3, 0, 20, 125};   // the range the MX rule produces
    int bad4 = 0;
    for (int ei = 0; ei < 7; ++ei) {
      const int e = exps[ei];
      const float s = e == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(e + 127) << 23);
      for (int v = 1; v < 256; ++v) {
        const int u = ((v ^ l) & 255) | 1;           // nonzero: -0 and +0 codes need no care
        const float x0 = (l & 1 ? -1.f : 1.f) * ((float)v / 32.f) * s;
        const float x1 = (l & 2 ? -1.f : 1.f) * ((float)u / 32.f) * s;
        const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x0, x1, s, 1);
        const uint32_t want = (e2m1_encode(x0, s) | (e2m1_encode(x1, s) << 4)) << 8;
        bad4 += w != want;
      }
    }
    atomicAdd(&counts[8], bad4);
  }

  {  // 32x32x16 bf16
    bf16x8_t a, b;
    for (int t = 0; t < 8; ++t) {
      a[t] = (__bf16)(float)st_a(l % 32, 8 * (l / 32) + t);
      b[t] = (__bf16)(float)st_b(8 * (l / 32) + t, l % 32);
    }
    f32x16_t d = {};
    d = mfma32_bf16(a, b, d);
    int bad = 0;
    for (int j = 0; j < 16; ++j) {
      const int m = 8 * (j / 4) + 4 * (l / 32) + (j % 4), n = l % 32;
      int ref = 0;
      for (int kk = 0; kk < 16; ++kk) ref += st_a(m, kk) * st_b(kk, n);
      bad += d[j] != (float)ref;
    }
    atomicAdd(&counts[2], bad);
  }
  {  // 16x16x32 bf16 and fp16
    bf16x8_t a, b;
    f16x8_t ah, bh;
    for (int t = 0; t < 8; ++t) {
      const float av = (float)st_a(l % 16, 8 * (l / 16) + t);
      const float bv = (float)st_b(8 * (l / 16) + t, l % 16);
      a[t] = (__bf16)av; b[t] = (__bf16)bv;
      ah[t] = (_Float16)av; bh[t] = (_Float16)bv;
    }
    f32x4_t d = {}, dh = {};
    d = mfma16_bf16(a, b, d);
    dh = mfma16_f16(ah, bh, dh);
    int bad = 0, badh = 0;
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * (l / 16) + j, n = l % 16;
      int ref = 0;
      for (int kk = 0; kk < 32; ++kk) ref += st_a(m, kk) * st_b(kk, n);
      bad += d[j] != (float)ref;
      badh += dh[j] != (float)ref;
    }
    atomicAdd(&counts[3], bad);
    atomicAdd(&counts[4], badh);
  }
}

__global__ void k_zero_i32(int32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

int selftest_count() { return ST_COUNT; }

hipError_t launch_selftest(int32_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, stream, counts, ST_COUNT);
  hipLaunchKernelGGL(k_selftest, dim3(1), dim3(64), 0, stream, counts);
  return hipGetLastError();
}

}  // namespace csa2
