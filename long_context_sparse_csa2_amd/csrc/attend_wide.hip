// Steps a8 + a9 for many queries at once (prefill): one 512-thread
// workgroup per query covering all 64 heads, so every gathered row is read
// and dequantised once for the whole query.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: each query attends to
// its selected main-KV entries plus the layer's SWA rows, the 512-d latent
// being both key and value; section 2.4.4: FP4 main KV dequantised before
// attention, FP8 SWA KV.
//
// Per 64-row chunk (main-KV chunks first, then SWA chunks, so each chunk has
// one row type):
//   raw     the chunk's row bytes (288 B main, 512 B SWA), prefetched into
//           registers one chunk ahead and written to LDS
//   S       64 heads x 64 rows, bf16 MFMA 16x16x32; wave w = (head group
//           w & 3, row half w >> 2), query tile in registers
//   V^T     fp16 [512 dims][64 rows] staged from the raw bytes
//   softmax running max per head shared through LDS; each wave keeps the
//           sum of its own rows (same reference max), added at the end
//   O += P V  fp16 MFMA 16x16x32; wave w = (head group, 256-dim half)
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int AW_ROWS = 64;            // rows per chunk
constexpr int AW_THREADS = 512;
constexpr int AW_RAW = 528;            // LDS bytes per raw row (>= 512 + padding)
constexpr int AW_PAD = 8;              // fp16 padding of vt / pl rows
constexpr int AW_MAX_SWA = 128;       // largest SWA window per query

__global__ __launch_bounds__(AW_THREADS, 1) void k_attend_wide(
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa_codes,
    const float* __restrict__ swa_scale, int64_t T_swa, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t raw[AW_ROWS * AW_RAW];
  __shared__ __align__(16) _Float16 vt[D_LAT][AW_ROWS + AW_PAD];
  __shared__ __align__(16) _Float16 pl[H_ATT][AW_ROWS + AW_PAD];
  __shared__ int64_t rowoff[AW_ROWS];
  __shared__ float rowsig[AW_ROWS];
  __shared__ int64_t nrowoff[AW_ROWS];
  __shared__ float nrowsig[AW_ROWS];
  __shared__ float red_m[2][H_ATT];
  __shared__ float red_l[2][H_ATT];

  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, qd = lane >> 4;
  const int hg = wave & 3, half = wave >> 2;
  const int64_t seq = q_seq[q];
  const int64_t sst = swa_start[q];
  int64_t sl64 = swa_len[q];
  if (sst < 0 || sst >= T_swa) sl64 = 0;
  else if (sl64 > T_swa - sst) sl64 = T_swa - sst;
  const int sl = sl64 < 0 ? 0 : (sl64 > AW_MAX_SWA ? AW_MAX_SWA : (int)sl64);
  const int nmc = (k + AW_ROWS - 1) / AW_ROWS;
  const int nch = nmc + (sl + AW_ROWS - 1) / AW_ROWS;

  // the row list of chunk ch: offsets (-1 = masked) and SWA scales
  auto row_info = [&](int ch, int r, int64_t& off, float& sg) __attribute__((always_inline)) {
    off = -1;
    sg = 1.f;
    if (ch < nmc) {
      const int rr = ch * AW_ROWS + r;
      if (rr < k) {
        const int e = idx[(int64_t)q * k + rr];
        if (e >= 0) off = seq * cap + e;
      }
    } else {
      const int rr = (ch - nmc) * AW_ROWS + r;
      if (rr < sl) {
        off = seq * T_swa + sst + rr;
        sg = swa_scale[off];
      }
    }
  };
  // this thread's share of a chunk's raw bytes: row tid >> 3, part tid & 7
  const int pr = tid >> 3, pp = tid & 7;
  u32x4_t pf0 = {0u, 0u, 0u, 0u}, pf1 = pf0, pf2 = pf0, pf3 = pf0;
  auto prefetch = [&](bool main_rows, int64_t off) __attribute__((always_inline)) {
    if (off < 0) return;
    const uint8_t* base = main_rows ? kv_codes + off * 256 + pp * 32 : swa_codes + off * 512 + pp * 64;
    pf0 = *(const u32x4_t*)base;
    pf1 = *(const u32x4_t*)(base + 16);
    // main rows: 16 scale bytes (used by pp < 2); SWA rows: the part's next 32 B
    pf2 = *(const u32x4_t*)(main_rows ? kv_scales + off * 32 + (pp & 1) * 16 : base + 32);
    if (!main_rows) pf3 = *(const u32x4_t*)(base + 48);
  };
  auto stash = [&](bool main_rows, int64_t off) __attribute__((always_inline)) {
    if (off < 0) return;
    uint8_t* dst = raw + pr * AW_RAW;
    if (main_rows) {
      *(u32x4_t*)(dst + pp * 32) = pf0;
      *(u32x4_t*)(dst + pp * 32 + 16) = pf1;
      if (pp < 2) *(u32x4_t*)(dst + 256 + pp * 16) = pf2;
    } else {
      u32x4_t* d = (u32x4_t*)(dst + pp * 64);
      d[0] = pf0;
      d[1] = pf1;
      d[2] = pf2;
      d[3] = pf3;
    }
  };

  // query tile of head group hg: head 16hg + r16, dims 128qd + 8s .. +7
  bf16x8_t a[16];
  {
    const uint16_t* qp = qv + ((int64_t)q * H_ATT + hg * 16 + r16) * D_LAT + qd * 128;
#pragma unroll
    for (int s = 0; s < 16; ++s) a[s] = *(const bf16x8_t*)(qp + 8 * s);
  }
  f32x4_t o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; }

  if (nch > 0) {
    if (tid < AW_ROWS) row_info(0, tid, nrowoff[tid], nrowsig[tid]);
    __syncthreads();
    prefetch(0 < nmc, nrowoff[pr]);
  }

  for (int ch = 0; ch < nch; ++ch) {
    const bool is_main = ch < nmc;
    // ---- this chunk's rows into LDS; next chunk's row list; its bytes in flight
    if (tid < AW_ROWS) { rowoff[tid] = nrowoff[tid]; rowsig[tid] = nrowsig[tid]; }
    stash(is_main, nrowoff[pr]);
    __syncthreads();
    if (ch + 1 < nch && tid < AW_ROWS) row_info(ch + 1, tid, nrowoff[tid], nrowsig[tid]);
    __syncthreads();
    if (ch + 1 < nch) prefetch(ch + 1 < nmc, nrowoff[pr]);

    // ---- S = Q K^T: rows 32*half .. +31 (two 16-row tiles), heads of group hg
    f32x4_t sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = half * 32 + rt * 16 + r16;
      const uint8_t* rp = raw + row * AW_RAW;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if (is_main) {
        const u32x4_t* cw = (const u32x4_t*)(rp + qd * 64);
        const u32x4_t w0 = cw[0], w1 = cw[1], w2 = cw[2], w3 = cw[3];
        const uint64_t sc = *(const uint64_t*)(rp + 256 + qd * 8);
        const u32x4_t wq[4] = {w0, w1, w2, w3};
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const float scl = e4m3_val((uint32_t)(sc >> (8 * (s >> 1))) & 0xFFu);
          acc = mfma16_bf16(a[s], fp4x8_to_bf16_scaled(wq[s >> 2][s & 3], scl), acc);
        }
      } else {
        const u32x4_t* cw = (const u32x4_t*)(rp + qd * 128);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const u32x4_t wv = cw[s2];
          acc = mfma16_bf16(a[2 * s2], fp8x8_to_bf16(wv[0], wv[1]), acc);
          acc = mfma16_bf16(a[2 * s2 + 1], fp8x8_to_bf16(wv[2], wv[3]), acc);
        }
        const float sg = rowsig[row];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= sg;
      }
      if (rowoff[row] < 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = -INFINITY;
      }
      sacc[rt] = acc;
    }

    // ---- V^T (fp16): thread owns rows 2rp2, 2rp2+1 and dims 32db .. +31
    {
      const int rp2 = tid & 31, db = tid >> 5;
      const int64_t off0 = rowoff[2 * rp2], off1 = rowoff[2 * rp2 + 1];
      const uint8_t* r0 = raw + (2 * rp2) * AW_RAW;
      const uint8_t* r1 = r0 + AW_RAW;
      _Float16* vcol = &vt[db * 32][2 * rp2];
      auto put8 = [&](int dim0, f16x8_t x0, f16x8_t x1) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          f16x2_t pr2;
          pr2[0] = off0 >= 0 ? x0[b] : (_Float16)0.f;
          pr2[1] = off1 >= 0 ? x1[b] : (_Float16)0.f;
          *(f16x2_t*)(vcol + (dim0 + b) * (AW_ROWS + AW_PAD)) = pr2;
        }
      };
      if (is_main) {
        const u32x4_t c0 = *(const u32x4_t*)(r0 + db * 16), c1 = *(const u32x4_t*)(r1 + db * 16);
        const uint32_t s0 = *(const uint16_t*)(r0 + 256 + db * 2);
        const uint32_t s1 = *(const uint16_t*)(r1 + 256 + db * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)          // 8 dims per word, 2 words per scale group
          put8(8 * i, fp4x8_to_f16_scaled(c0[i], e4m3_val((s0 >> (8 * (i >> 1))) & 0xFFu)),
               fp4x8_to_f16_scaled(c1[i], e4m3_val((s1 >> (8 * (i >> 1))) & 0xFFu)));
      } else {
        const float g0 = rowsig[2 * rp2], g1 = rowsig[2 * rp2 + 1];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const u32x4_t x0 = *(const u32x4_t*)(r0 + db * 32 + 16 * i2);
          const u32x4_t x1 = *(const u32x4_t*)(r1 + db * 32 + 16 * i2);
          put8(16 * i2, fp8x8_to_f16_scaled(x0[0], x0[1], g0), fp8x8_to_f16_scaled(x1[0], x1[1], g1));
          put8(16 * i2 + 8, fp8x8_to_f16_scaled(x0[2], x0[3], g0),
               fp8x8_to_f16_scaled(x1[2], x1[3], g1));
        }
      }
    }

    // ---- online softmax: chunk max per head over both row halves
    float cm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = fmaxf(sacc[0][j], sacc[1][j]);
      v = fmaxf(v, __shfl_xor(v, 1));
      v = fmaxf(v, __shfl_xor(v, 2));
      v = fmaxf(v, __shfl_xor(v, 4));
      v = fmaxf(v, __shfl_xor(v, 8));
      cm[j] = v;
    }
    if (r16 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) red_m[half][hg * 16 + 4 * qd + j] = cm[j];
    }
    __syncthreads();
    float alpha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = hg * 16 + 4 * qd + j;
      const float m_new = fmaxf(m_run[j], fmaxf(red_m[0][hh], red_m[1][hh]));
      float psum = 0.f;
      if (m_new == -INFINITY) {
        alpha[j] = 1.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) pl[hh][half * 32 + rt * 16 + r16] = (_Float16)0.f;
      } else {
        alpha[j] = expf(m_run[j] - m_new);          // 0 when m_run is -inf
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const float p = expf(sacc[rt][j] - m_new); // masked rows: exp(-inf) = 0
          psum += p;
          pl[hh][half * 32 + rt * 16 + r16] = (_Float16)p;
        }
      }
      psum += __shfl_xor(psum, 1);
      psum += __shfl_xor(psum, 2);
      psum += __shfl_xor(psum, 4);
      psum += __shfl_xor(psum, 8);
      l_run[j] = l_run[j] * alpha[j] + psum;        // this wave's rows only
      m_run[j] = m_new;
    }
    __syncthreads();

    // ---- O += P V: heads of group hg, dims 256*half .. +255 (16 tiles)
    // (the O rows of this lane are the same heads as its S rows: 16hg + 4qd + j)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[t][j] *= alpha[j];
    }
    const f16x8_t pa0 = *(const f16x8_t*)&pl[hg * 16 + r16][qd * 8];
    const f16x8_t pa1 = *(const f16x8_t*)&pl[hg * 16 + r16][32 + qd * 8];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int dim = half * 256 + 16 * t + r16;
      const f16x8_t vb0 = *(const f16x8_t*)&vt[dim][qd * 8];
      const f16x8_t vb1 = *(const f16x8_t*)&vt[dim][32 + qd * 8];
      o[t] = mfma16_f16(pa0, vb0, o[t]);
      o[t] = mfma16_f16(pa1, vb1, o[t]);
    }
  }

  // ---- totals: the two row-half waves of a head group hold partial sums
  if (r16 == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red_l[half][hg * 16 + 4 * qd + j] = l_run[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = hg * 16 + 4 * qd + j;
    const float L = red_l[0][hh] + red_l[1][hh];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* op = out + ((int64_t)q * H_ATT + hh) * D_LAT + half * 256 + r16;
#pragma unroll
    for (int t = 0; t < 16; ++t) op[16 * t] = o[t][j] * inv;
    if (lse && half == 0 && r16 == 0)
      lse[(int64_t)q * H_ATT + hh] = L > 0.f ? m_run[j] + logf(L) : -INFINITY;
  }
}

hipError_t launch_attend_wide(const uint16_t* q, const int32_t* q_seq, int Q,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
                              const int32_t* idx, int k, const uint8_t* swa_codes,
                              const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                              const int32_t* swa_len, float* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(k_attend_wide, dim3((unsigned)Q), dim3(AW_THREADS), 0, stream, q, q_seq,
                     kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale, T_swa, swa_start,
                     swa_len, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
