// Steps a1-a3: m-to-1 softmax pooling, FP4 main-KV quantisation, indexer-K
// projection and MXFP4 quantisation, one workgroup per 32 entries.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: non-overlapping
// compression, indexer K projected from the main-KV entry; section 2.4.4:
// E2M1 + one E4M3 scale per 16 channels for main KV, OCP MXFP4 for indexer K.
// The per-channel softmax pooling form follows the mer.dev commentary,
// section 4.1.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int CQ_ENT = 32;          // entries per workgroup
constexpr int CQ_XPAD = 8;          // bf16 padding of an LDS latent row
constexpr int CQ_KPAD = 4;          // fp32 padding of an LDS indexer-K row

// APPEND = false: entry j of sequence b pools rows jm .. jm + m - 1 of
// h[b] / z[b] ([B][T][512]) and is written at entry e0 + j.
// APPEND = true (decode-time append, one workgroup per sequence, n_ent = 1):
// the token count n_tok[b] says whether the new token (row b of h_new /
// z_new) completes a group of m; if it does, the group is the m - 1 tokens
// waiting in the tail (h / z as [B][m - 1][512]) followed by the new one,
// and it becomes entry (n_tok[b] + 1) / m - 1.  Nothing is written when no
// group completes or the entry would fall at or past cap.
template <bool APPEND>
__global__ __launch_bounds__(256) void k_compress_quant(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ z, int64_t T, int m,
    int64_t n_ent, const uint16_t* __restrict__ w_ik, uint8_t* __restrict__ kv_codes,
    uint8_t* __restrict__ kv_scales, uint8_t* __restrict__ ik_codes,
    uint8_t* __restrict__ ik_scales, int64_t cap, int64_t e0,
    const uint16_t* __restrict__ h_new, const uint16_t* __restrict__ z_new,
    const int64_t* __restrict__ n_tok) {
  __shared__ __align__(16) uint16_t xs[CQ_ENT][D_LAT + CQ_XPAD];   // dequantised main KV, bf16
  __shared__ __align__(16) float ks[CQ_ENT][D_IDX + CQ_KPAD];      // projected indexer K

  const int b = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * CQ_ENT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (APPEND) {
    const int64_t t = n_tok[b];                    // tokens before the new one
    if ((t + 1) % m != 0 || (t + 1) / m > cap) return;
    e0 = (t + 1) / m - 1;
  }
  // raw row t (< m) of entry j
  auto hrow = [&](int64_t j, int t) -> const uint16_t* {
    if constexpr (APPEND)
      return t == m - 1 ? h_new + (int64_t)b * D_LAT : h + ((int64_t)b * (m - 1) + t) * D_LAT;
    else
      return h + ((int64_t)b * T + j * m + t) * D_LAT;
  };
  auto zrow = [&](int64_t j, int t) -> const uint16_t* {
    if constexpr (APPEND)
      return t == m - 1 ? z_new + (int64_t)b * D_LAT : z + ((int64_t)b * (m - 1) + t) * D_LAT;
    else
      return z + ((int64_t)b * T + j * m + t) * D_LAT;
  };

  // ---- phase 1: pooling + main-KV quantisation; wave w owns entries 8w..8w+7,
  //      lane l owns channels 8l..8l+7 (two lanes per 16-channel scale group).
  for (int i = 0; i < 8; ++i) {
    const int jl = wave * 8 + i;
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
  }
  __syncthreads();

  // ---- phase 2: k[32 entries][128] = xhat[32][512] . w_ik^T with 32x32x16 bf16
  //      MFMA; wave w computes output dims 32w..32w+31.
  {
    const int r = lane & 31, kh = lane >> 5;
    const uint16_t* wrow = w_ik + (int64_t)(wave * 32 + r) * D_LAT + kh * 8;
    f32x16_t acc = {};
#pragma unroll 8
    for (int s = 0; s < D_LAT / 16; ++s) {
      const bf16x8_t a = *(const bf16x8_t*)&xs[r][16 * s + kh * 8];
      const bf16x8_t bb = *(const bf16x8_t*)(wrow + 16 * s);
      acc = mfma32_bf16(a, bb, acc);
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) ks[8 * (jj >> 2) + 4 * kh + (jj & 3)][wave * 32 + r] = acc[jj];
  }
  __syncthreads();

  // ---- phase 3: MXFP4, one (entry, 32-dim group) per thread pair, 16 dims each
  {
    const int tid = threadIdx.x;
    const int task = tid >> 1, sub = tid & 1;
    const int jl = task >> 2, g = task & 3;
    const int64_t j = j0 + jl;
    float v[16];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      v[c] = ks[jl][g * 32 + sub * 16 + c];
      amax = fmaxf(amax, fabsf(v[c]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    int E = -127;
    if (amax > 0.f) {
      int ex;
      (void)frexpf(amax, &ex);       // floor(log2 amax) = ex - 1
      E = ex - 1 - 2;                 // minus emax of E2M1
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    uint64_t word = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t n = amax > 0.f ? e2m1_encode(ldexpf(v[c], -E), 1.0f) : 0u;
      word |= (uint64_t)n << (4 * c);
    }
    if (j < n_ent) {
      const int64_t ent = (int64_t)b * cap + e0 + j;
      *(uint64_t*)(ik_codes + ent * 64 + g * 16 + sub * 8) = word;
      if (sub == 0) ik_scales[ent * 4 + g] = (uint8_t)(E + 127);
    }
  }
}

hipError_t launch_compress_quant(const uint16_t* h, const uint16_t* z, int B, int64_t T, int m,
                                 const uint16_t* w_ik, uint8_t* kv_codes, uint8_t* kv_scales,
                                 uint8_t* ik_codes, uint8_t* ik_scales, int64_t cap, int64_t e0,
                                 hipStream_t stream) {
  const int64_t n_ent = T / m;
  const dim3 grid((unsigned)((n_ent + CQ_ENT - 1) / CQ_ENT), (unsigned)B);
  hipLaunchKernelGGL(k_compress_quant<false>, grid, dim3(256), 0, stream, h, z, T, m, n_ent, w_ik,
                     kv_codes, kv_scales, ik_codes, ik_scales, cap, e0, nullptr, nullptr,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_append_compress(const uint16_t* h_new, const uint16_t* z_new, int B, int m,
                                  const uint16_t* tail_h, const uint16_t* tail_z,
                                  const int64_t* n_tok, const uint16_t* w_ik, uint8_t* kv_codes,
                                  uint8_t* kv_scales, uint8_t* ik_codes, uint8_t* ik_scales,
                                  int64_t cap, hipStream_t stream) {
  hipLaunchKernelGGL(k_compress_quant<true>, dim3(1, (unsigned)B), dim3(256), 0, stream, tail_h,
                     tail_z, (int64_t)m, m, (int64_t)1, w_ik, kv_codes, kv_scales, ik_codes,
                     ik_scales, cap, (int64_t)0, h_new, z_new, n_tok);
  return hipGetLastError();
}

}  // namespace csa2
