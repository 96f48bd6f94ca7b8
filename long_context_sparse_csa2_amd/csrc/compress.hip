// Steps a1-a3: m-to-1 softmax pooling, FP4 main-KV quantisation, indexer-K
// projection and MXFP4 quantisation, one workgroup per 8 entries; and the
// decode-time append, which runs the same steps on the group a new token
// completes.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: non-overlapping
// compression, indexer K projected from the main-KV entry; section 2.4.4:
// E2M1 + one E4M3 scale per 16 channels for main KV, OCP MXFP4 for indexer K.
// The per-channel softmax pooling form follows the mer.dev commentary,
// section 4.1.
#include "common.h"
#include "launch.h"

namespace csa2 {

// Entries per workgroup of the batch compressor.  A small launch takes 8
// (two per wave): each wave's pooling and quantisation are serial work, and
// more workgroups cover the device (4,096 entries at m = 2 on MI355X: 44 us
// with 32 per workgroup, 30 with 16, 28 with 8).  A launch that fills the
// device with 32 per workgroup keeps 32: every workgroup reads the whole
// 128 KB projection matrix, so 8 per workgroup quadruples that traffic
// (4 x 2^20 entries at m = 1: 1.30 ms with 32, 1.95 ms with 8).
constexpr int CQ_ENT_SMALL = 8, CQ_ENT_LARGE = 32;
constexpr int64_t CQ_LARGE_WGS = 1024;
constexpr int CQ_XPAD = 8;          // bf16 padding of an LDS latent row
constexpr int CQ_KPAD = 4;          // fp32 padding of an LDS indexer-K row

// Phase 1 of the compressor for a wave's E entries when an entry has M <= 2
// raw rows: every row is requested first, then each entry is pooled (per
// channel, softmax over the M rows of z weighting the rows of h; M == 1:
// the row itself) and handed to quant(x, jl, j).  Entries past n_ent get
// zero rows in xs and nothing stored.
template <int M, int E, typename HRow, typename ZRow, typename Quant>
__device__ __forceinline__ void pool_rows(HRow hrow, ZRow zrow, int64_t n_ent, int64_t j0,
                                          int wave, int lane, Quant quant,
                                          uint16_t (*xs)[D_LAT + CQ_XPAD]) {
  u32x4_t hv[E][M], zv[E][M];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t jr = j0 + wave * E + i;
    const int64_t j = jr < n_ent ? jr : n_ent - 1;
#pragma unroll
    for (int t = 0; t < M; ++t) {
      hv[i][t] = *(const u32x4_t*)(hrow(j, t) + lane * 8);
      if (M > 1) zv[i][t] = *(const u32x4_t*)(zrow(j, t) + lane * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int jl = wave * E + i;
    const int64_t j = j0 + jl;
    float x[8];
    if constexpr (M == 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[2 * c] = __uint_as_float(hv[i][0][c] << 16);
        x[2 * c + 1] = __uint_as_float(hv[i][0][c] & 0xFFFF0000u);
      }
    } else {
      float zmax[8], num[8], den[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) { zmax[c] = -INFINITY; num[c] = 0.f; den[c] = 0.f; }
#pragma unroll
      for (int t = 0; t < M; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          zmax[2 * c] = fmaxf(zmax[2 * c], __uint_as_float(zv[i][t][c] << 16));
          zmax[2 * c + 1] = fmaxf(zmax[2 * c + 1], __uint_as_float(zv[i][t][c] & 0xFFFF0000u));
        }
#pragma unroll
      for (int t = 0; t < M; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float e0v = expf(__uint_as_float(zv[i][t][c] << 16) - zmax[2 * c]);
          const float e1v = expf(__uint_as_float(zv[i][t][c] & 0xFFFF0000u) - zmax[2 * c + 1]);
          num[2 * c] += e0v * __uint_as_float(hv[i][t][c] << 16);
          num[2 * c + 1] += e1v * __uint_as_float(hv[i][t][c] & 0xFFFF0000u);
          den[2 * c] += e0v;
          den[2 * c + 1] += e1v;
        }
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = num[c] / den[c];
    }
    if (j < n_ent) quant(x, jl, j);                     // uniform per wave
    else *(u32x4_t*)&xs[jl][lane * 8] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// The compressor for entries j0 .. j0 + ENT - 1 of sequence b (those below
// n_ent), written at entries e0 + j.  hrow(j, t) / zrow(j, t) give raw row
// t (< m) of entry j.  ONE_ENTRY (the decode append, one valid entry, ENT =
// 32) loads the whole projection operand at once instead of eight steps at
// a time.  With ENT < 32 the projection runs on 16x16x32 MFMAs whose rows
// past ENT are discarded.
template <bool ONE_ENTRY, int ENT, typename HRow, typename ZRow>
__device__ __forceinline__ void compress_entries(HRow hrow, ZRow zrow, int m, int64_t n_ent,
                                                 int64_t j0, int b, int64_t e0,
                                                 const uint16_t* __restrict__ w_ik,
                                                 uint8_t* __restrict__ kv_codes,
                                                 uint8_t* __restrict__ kv_scales,
                                                 uint8_t* __restrict__ ik_codes,
                                                 uint8_t* __restrict__ ik_scales, int64_t cap) {
  static_assert(ENT == 8 || ENT == 16 || ENT == 32, "8, 16 or 32 entries per workgroup");
  static_assert(!ONE_ENTRY || ENT == 32, "the append path keeps 32");
  constexpr int EPW = ENT / 4;                                     // entries per wave
  __shared__ __align__(16) uint16_t xs[ENT][D_LAT + CQ_XPAD];     // dequantised main KV, bf16
  __shared__ __align__(16) float ks[ENT][D_IDX + CQ_KPAD];        // projected indexer K
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the projection operand (wave w: output dims 32w..32w+31), for a single
  // entry loaded up front so that its latency overlaps the pooling
  const uint16_t* wrow = w_ik + (int64_t)(wave * 32 + (lane & 31)) * D_LAT + (lane >> 5) * 8;
  bf16x8_t wpre[ONE_ENTRY ? D_LAT / 16 : 1];
  if constexpr (ONE_ENTRY) {
#pragma unroll
    for (int s = 0; s < D_LAT / 16; ++s) wpre[s] = *(const bf16x8_t*)(wrow + 16 * s);
  }

  // ---- phase 1: pooling + main-KV quantisation; wave w owns entries EPW w ..,
  //      lane l owns channels 8l..8l+7 (two lanes per 16-channel scale group).
  // FP4 codes and E4M3 scales of entry j (local jl) from its pooled channels
  auto quantise = [&](const float (&x)[8], int jl, int64_t j) __attribute__((always_inline)) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(x[c]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const uint32_t sc = e4m3_encode_pos(amax / 6.0f);
    const float s = e4m3_val(sc);
    uint32_t word = 0;
    uint32_t xb[4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t n = sc == 0 ? 0u : e2m1_encode(x[c], s);
      word |= n << (4 * c);
      const uint32_t bits = bf16_bits_exact(e2m1_val(n) * s);
      if (c & 1) xb[c >> 1] |= bits << 16; else xb[c >> 1] = bits;
    }
    const int64_t ent = (int64_t)b * cap + e0 + j;
    *(uint32_t*)(kv_codes + ent * 256 + lane * 4) = word;
    // lanes 8i..8i+7 hold scale groups 4i..4i+3 (two lanes each)
    const uint32_t s1 = __shfl(sc, lane + 2), s2 = __shfl(sc, lane + 4), s3 = __shfl(sc, lane + 6);
    if ((lane & 7) == 0)
      *(uint32_t*)(kv_scales + ent * 32 + lane / 2) = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
    *(u32x4_t*)&xs[jl][lane * 8] = u32x4_t{xb[0], xb[1], xb[2], xb[3]};
  };
  if (!ONE_ENTRY && (m == 1 || m == 2)) {
    // the rows of all the wave's entries requested before any pooling (rows past
    // n_ent re-read the last entry; their results are not stored)
    if (m == 1) pool_rows<1, EPW>(hrow, zrow, n_ent, j0, wave, lane, quantise, xs);
    else pool_rows<2, EPW>(hrow, zrow, n_ent, j0, wave, lane, quantise, xs);
  } else {
    for (int i = 0; i < EPW; ++i) {
      const int jl = wave * EPW + i;
      const int64_t j = j0 + jl;
      if (j >= n_ent) {
        *(u32x4_t*)&xs[jl][lane * 8] = u32x4_t{0u, 0u, 0u, 0u};
        continue;
      }
      float x[8];
      if (m == 1) {
        const u32x4_t v = *(const u32x4_t*)(hrow(j, 0) + lane * 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[2 * c] = __uint_as_float(v[c] << 16);
          x[2 * c + 1] = __uint_as_float(v[c] & 0xFFFF0000u);
        }
      } else {
        float zmax[8], num[8], den[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) { zmax[c] = -INFINITY; num[c] = 0.f; den[c] = 0.f; }
        for (int t = 0; t < m; ++t) {
          const u32x4_t zv = *(const u32x4_t*)(zrow(j, t) + lane * 8);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            zmax[2 * c] = fmaxf(zmax[2 * c], __uint_as_float(zv[c] << 16));
            zmax[2 * c + 1] = fmaxf(zmax[2 * c + 1], __uint_as_float(zv[c] & 0xFFFF0000u));
          }
        }
        for (int t = 0; t < m; ++t) {
          const u32x4_t zv = *(const u32x4_t*)(zrow(j, t) + lane * 8);
          const u32x4_t hv = *(const u32x4_t*)(hrow(j, t) + lane * 8);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float e0v = expf(__uint_as_float(zv[c] << 16) - zmax[2 * c]);
            const float e1v = expf(__uint_as_float(zv[c] & 0xFFFF0000u) - zmax[2 * c + 1]);
            num[2 * c] += e0v * __uint_as_float(hv[c] << 16);
            num[2 * c + 1] += e1v * __uint_as_float(hv[c] & 0xFFFF0000u);
            den[2 * c] += e0v;
            den[2 * c + 1] += e1v;
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = num[c] / den[c];
      }
      quantise(x, jl, j);
    }
  }
  __syncthreads();

  // ---- phase 2: k[ENT entries][128] = xhat[ENT][512] . w_ik^T, wave w
  //      computing output dims 32w..32w+31: 32x32x16 bf16 MFMA for 32
  //      entries, two 16x16x32 column blocks for 8 or 16
  if constexpr (ENT <= 16) {
    const int r16 = lane & 15, kq = lane >> 4;
    const int ra = r16 < ENT ? r16 : 0;           // rows past ENT: any row, results unused
    const uint16_t* w0 = w_ik + (int64_t)(wave * 32 + r16) * D_LAT + kq * 8;
    const uint16_t* w1 = w0 + 16 * D_LAT;
    f32x4_t acc0 = {}, acc1 = {};
#pragma unroll 8
    for (int s = 0; s < D_LAT / 32; ++s) {
      const bf16x8_t a = *(const bf16x8_t*)&xs[ra][32 * s + kq * 8];
      acc0 = mfma16_bf16(a, *(const bf16x8_t*)(w0 + 32 * s), acc0);
      acc1 = mfma16_bf16(a, *(const bf16x8_t*)(w1 + 32 * s), acc1);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (4 * kq + jj < ENT) {
        ks[4 * kq + jj][wave * 32 + r16] = acc0[jj];
        ks[4 * kq + jj][wave * 32 + 16 + r16] = acc1[jj];
      }
    }
  } else {
    const int r = lane & 31, kh = lane >> 5;
    f32x16_t acc = {};
    if constexpr (ONE_ENTRY) {
#pragma unroll
      for (int s = 0; s < D_LAT / 16; ++s)
        acc = mfma32_bf16(*(const bf16x8_t*)&xs[r][16 * s + kh * 8], wpre[s], acc);
    } else {
#pragma unroll 8
      for (int s = 0; s < D_LAT / 16; ++s) {
        const bf16x8_t a = *(const bf16x8_t*)&xs[r][16 * s + kh * 8];
        const bf16x8_t bb = *(const bf16x8_t*)(wrow + 16 * s);
        acc = mfma32_bf16(a, bb, acc);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) ks[8 * (jj >> 2) + 4 * kh + (jj & 3)][wave * 32 + r] = acc[jj];
  }
  __syncthreads();

  // ---- phase 3: MXFP4, one (entry, 32-dim group) per TPT threads, VPT dims each
  {
    constexpr int TPT = 256 / (ENT * 4), VPT = 32 / TPT;
    const int tid = threadIdx.x;
    const int task = tid / TPT, sub = tid % TPT;
    const int jl = task >> 2, g = task & 3;
    const int64_t j = j0 + jl;
    float v[VPT];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
      v[c] = ks[jl][g * 32 + sub * VPT + c];
      amax = fmaxf(amax, fabsf(v[c]));
    }
#pragma unroll
    for (int o = 1; o < TPT; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int E = -127;
    if (amax > 0.f) {
      int ex;
      (void)frexpf(amax, &ex);       // floor(log2 amax) = ex - 1
      E = ex - 1 - 2;                 // minus emax of E2M1
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    // E2M1(v / 2^E), round to nearest even, saturating, by the gfx950 scaled
    // conversion (two values into byte sel of a word; it reads only the
    // exponent field of its scale, so 2^-127 goes in as the subnormal with
    // that field 0); an all-zero group stores +0 codes
    const float sc = __uint_as_float(E == -127 ? 0x00400000u : (uint32_t)(E + 127) << 23);
    uint32_t wd[2] = {0u, 0u};
#pragma unroll
    for (int c = 0; c < VPT; c += 8) {
      uint32_t x = 0u;
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[c], v[c + 1], sc, 0);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[c + 2 < VPT ? c + 2 : c], v[c + 3 < VPT ? c + 3 : c + 1], sc, 1);
      if constexpr (VPT >= 8) {
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[c + 4 < VPT ? c + 4 : c], v[c + 5 < VPT ? c + 5 : c], sc, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[c + 6 < VPT ? c + 6 : c], v[c + 7 < VPT ? c + 7 : c], sc, 3);
      }
      wd[c / 8] = amax > 0.f ? x : 0u;
    }
    const uint64_t word = (uint64_t)wd[0] | ((uint64_t)wd[1] << 32);
    if (j < n_ent) {
      const int64_t ent = (int64_t)b * cap + e0 + j;
      uint8_t* dst = ik_codes + ent * 64 + g * 16 + sub * (VPT / 2);
      if constexpr (VPT == 16) *(uint64_t*)dst = word;
      else if constexpr (VPT == 8) *(uint32_t*)dst = (uint32_t)word;
      else *(uint16_t*)dst = (uint16_t)word;
      if (sub == 0) ik_scales[ent * 4 + g] = (uint8_t)(E + 127);
    }
  }
}

template <int ENT>
__global__ __launch_bounds__(256) void k_compress_quant(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ z, int64_t T, int m,
    int64_t n_ent, const uint16_t* __restrict__ w_ik, uint8_t* __restrict__ kv_codes,
    uint8_t* __restrict__ kv_scales, uint8_t* __restrict__ ik_codes,
    uint8_t* __restrict__ ik_scales, int64_t cap, int64_t e0) {
  const int b = blockIdx.y;
  compress_entries<false, ENT>(
      [&](int64_t j, int t) { return h + ((int64_t)b * T + j * m + t) * D_LAT; },
      [&](int64_t j, int t) { return z + ((int64_t)b * T + j * m + t) * D_LAT; }, m, n_ent,
      (int64_t)blockIdx.x * ENT, b, e0, w_ik, kv_codes, kv_scales, ik_codes, ik_scales, cap);
}

hipError_t launch_compress_quant(const uint16_t* h, const uint16_t* z, int B, int64_t T, int m,
                                 const uint16_t* w_ik, uint8_t* kv_codes, uint8_t* kv_scales,
                                 uint8_t* ik_codes, uint8_t* ik_scales, int64_t cap, int64_t e0,
                                 hipStream_t stream) {
  const int64_t n_ent = T / m;
  const int64_t wgs_large = (n_ent + CQ_ENT_LARGE - 1) / CQ_ENT_LARGE * B;
  if (wgs_large >= CQ_LARGE_WGS) {
    const dim3 grid((unsigned)((n_ent + CQ_ENT_LARGE - 1) / CQ_ENT_LARGE), (unsigned)B);
    hipLaunchKernelGGL(k_compress_quant<CQ_ENT_LARGE>, grid, dim3(256), 0, stream, h, z, T, m,
                       n_ent, w_ik, kv_codes, kv_scales, ik_codes, ik_scales, cap, e0);
  } else {
    const dim3 grid((unsigned)((n_ent + CQ_ENT_SMALL - 1) / CQ_ENT_SMALL), (unsigned)B);
    hipLaunchKernelGGL(k_compress_quant<CQ_ENT_SMALL>, grid, dim3(256), 0, stream, h, z, T, m,
                       n_ent, w_ik, kv_codes, kv_scales, ik_codes, ik_scales, cap, e0);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ decode append
// Decode-time append: the per-sequence state block of the V4 KV layout
// ("DeepSeek-V4" page, Fig. 6: a fixed-size block per request holding the
// SWA entries of the most recent tokens and the uncompressed tail that is
// not yet ready for compression).  One workgroup per sequence, one token:
//   - with t = n_tok[b] tokens before it, the new token completes a group of
//     m iff (t + 1) % m == 0; then the m - 1 tail tokens followed by the new
//     one are compressed exactly as above into entry (t + 1) / m - 1 (not
//     written at or past cap);
//   - otherwise the token's raw latent and logits go to tail slot t % m;
//   - its SWA latent x becomes one FP8 row in ring slot t % W: sigma =
//     max|x| / 448 and codes E4M3FN(x / sigma), both quotients IEEE fp32
//     (all-zero row: sigma = 0, +0 codes);
//   - the next query's geometry is written and the count advances.
__device__ __forceinline__ void append_state_wave(
    int64_t t, int b, const uint16_t* __restrict__ h_new, const uint16_t* __restrict__ z_new,
    const uint16_t* __restrict__ swa_new, int m, uint16_t* __restrict__ tail_h,
    uint16_t* __restrict__ tail_z, int64_t* __restrict__ n_tok, uint8_t* __restrict__ swa_codes,
    float* __restrict__ swa_scale, int64_t W, int64_t* __restrict__ n_vis,
    int64_t* __restrict__ swa_start, int32_t* __restrict__ swa_len) {
  const int lane = threadIdx.x & 63;                  // lane l owns channels 8l .. 8l + 7
  const int s = (int)(t % m);
  if (s < m - 1) {                                    // the group is not complete: keep the token
    const int64_t src = (int64_t)b * D_LAT + lane * 8;
    const int64_t dst = ((int64_t)b * (m - 1) + s) * D_LAT + lane * 8;
    *(u32x4_t*)(tail_h + dst) = *(const u32x4_t*)(h_new + src);
    *(u32x4_t*)(tail_z + dst) = *(const u32x4_t*)(z_new + src);
  }
  if (W > 0) {
    const u32x4_t v = *(const u32x4_t*)(swa_new + (int64_t)b * D_LAT + lane * 8);
    float x[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[2 * c] = __uint_as_float(v[c] << 16);
      x[2 * c + 1] = __uint_as_float(v[c] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(x[c]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sig = amax / 448.0f;                  // IEEE division, as every quotient here
    uint32_t lo = 0, hi = 0;
    if (sig > 0.f) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float q = x[c] / sig;
        const uint32_t code = e4m3_encode_pos(fabsf(q)) | (q < 0.f ? 0x80u : 0u);
        if (c < 4) lo |= code << (8 * c); else hi |= code << (8 * (c - 4));
      }
    }
    const int64_t slot = (int64_t)b * W + t % W;
    *(uint2*)(swa_codes + slot * D_LAT + lane * 8) = make_uint2(lo, hi);
    if (lane == 0) swa_scale[slot] = sig;
  }
  if (lane == 0) {
    const int64_t n = t + 1;
    const int64_t len = n < W ? n : W;
    if (n_vis) n_vis[b] = n / m;
    if (swa_start) swa_start[b] = W > 0 ? (n - len) % W : 0;
    if (swa_len) swa_len[b] = (int32_t)len;
    n_tok[b] = n;
  }
}

__global__ __launch_bounds__(256) void k_append(
    const uint16_t* __restrict__ h_new, const uint16_t* __restrict__ z_new,
    const uint16_t* __restrict__ swa_new, int m, uint16_t* __restrict__ tail_h,
    uint16_t* __restrict__ tail_z, int64_t* __restrict__ n_tok, const uint16_t* __restrict__ w_ik,
    uint8_t* __restrict__ kv_codes, uint8_t* __restrict__ kv_scales,
    uint8_t* __restrict__ ik_codes, uint8_t* __restrict__ ik_scales, int64_t cap,
    uint8_t* __restrict__ swa_codes, float* __restrict__ swa_scale, int64_t W,
    int64_t* __restrict__ n_vis, int64_t* __restrict__ swa_start, int32_t* __restrict__ swa_len) {
  const int b = blockIdx.x;
  const int64_t t = n_tok[b];                         // tokens before the new one
  __syncthreads();                                    // read by every thread before it changes
  // the last wave files the token (its loads overlap the compressor's)
  if (threadIdx.x >= 192)
    append_state_wave(t, b, h_new, z_new, swa_new, m, tail_h, tail_z, n_tok, swa_codes,
                      swa_scale, W, n_vis, swa_start, swa_len);
  if ((t + 1) % m == 0 && (t + 1) / m <= cap) {
    const uint16_t* th = tail_h;
    const uint16_t* tz = tail_z;
    compress_entries<true, 32>(
        [&](int64_t, int r) {
          return r == m - 1 ? h_new + (int64_t)b * D_LAT : th + ((int64_t)b * (m - 1) + r) * D_LAT;
        },
        [&](int64_t, int r) {
          return r == m - 1 ? z_new + (int64_t)b * D_LAT : tz + ((int64_t)b * (m - 1) + r) * D_LAT;
        },
        m, (int64_t)1, (int64_t)0, b, (t + 1) / m - 1, w_ik, kv_codes, kv_scales, ik_codes,
        ik_scales, cap);
  }
}

hipError_t launch_append(const uint16_t* h_new, const uint16_t* z_new, const uint16_t* swa_new,
                         int B, int m, uint16_t* tail_h, uint16_t* tail_z, int64_t* n_tok,
                         const uint16_t* w_ik, uint8_t* kv_codes, uint8_t* kv_scales,
                         uint8_t* ik_codes, uint8_t* ik_scales, int64_t cap, uint8_t* swa_codes,
                         float* swa_scale, int64_t W, int64_t* n_vis, int64_t* swa_start,
                         int32_t* swa_len, hipStream_t stream) {
  hipLaunchKernelGGL(k_append, dim3((unsigned)B), dim3(256), 0, stream, h_new, z_new, swa_new, m,
                     tail_h, tail_z, n_tok, w_ik, kv_codes, kv_scales, ik_codes, ik_scales, cap,
                     swa_codes, swa_scale, W, n_vis, swa_start, swa_len);
  return hipGetLastError();
}

}  // namespace csa2
