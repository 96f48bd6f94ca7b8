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
//   staging  thread t holds the raw bytes of row t & 63, dims 64 (t >> 6)
//            .. +63, loaded one chunk ahead (the row ids two chunks ahead),
//            and writes them dequantised to fp16 in LDS (attend_stage.h)
//   S        64 heads x 64 rows, fp16 MFMA 16x16x32; wave w = (head group
//            w & 3, row half w >> 2); the query tile sits in registers as
//            fp16, each head scaled by a power of two (undone on S)
//   softmax  running max per head shared through LDS; each wave keeps the
//            sum of its own rows (same reference max), added at the end; the
//            reference max only moves when a chunk beats it by more than
//            e^8, so the rescaling of O is skipped in most chunks
//   O += P V fp16 MFMA 16x16x32; wave w = (head group, 256-dim half); V
//            columns through transposing LDS reads of the staged rows
#include "common.h"
#include "launch.h"
#include "attend_stage.h"

namespace csa2 {

constexpr int AW_THREADS = 512;
constexpr int AW_PAD = 8;              // fp16 padding of pl rows
constexpr int AW_MAX_SWA = 128;        // largest SWA window per query
constexpr float AW_LAZY = 8.f;         // slack of the softmax reference max (natural log)

__global__ __launch_bounds__(AW_THREADS, 1) void k_attend_wide(
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa_codes,
    const float* __restrict__ swa_scale, int64_t T_swa, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float* __restrict__ out, float* __restrict__ lse,
    RopeArgs rp) {
  __shared__ __align__(16) _Float16 kv[2][CH_ROWS * KV_LD];        // K (+ V of main rows), V of SWA rows
  __shared__ __align__(16) _Float16 pl[H_ATT][CH_ROWS + AW_PAD];  // P of the chunk
  __shared__ int64_t rowoff[CH_ROWS];
  __shared__ float rowsig[CH_ROWS];
  __shared__ float red_m[2][H_ATT];
  __shared__ float red_l[2][H_ATT];
  __shared__ f32x2_t rcs[ROPE_MAX_PAIRS];                          // RoPE (cos, sin) per pair

  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, qd = lane >> 4;
  const int hg = wave & 3, half = wave >> 2;
  const int64_t seq = q_seq[q];
  const int64_t sst = swa_start[q];
  int64_t sl64 = swa_len[q];
  if (sst < 0 || sst >= T_swa) sl64 = 0;                     // ring: start must be a slot
  else if (sl64 > T_swa) sl64 = T_swa;                       // at most one lap
  const int sl = sl64 < 0 ? 0 : (sl64 > AW_MAX_SWA ? AW_MAX_SWA : (int)sl64);
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  const int nch = nmc + (sl + CH_ROWS - 1) / CH_ROWS;
  const int srow = tid & 63, spart = tid >> 6;          // this thread's staging share

  // selected entry of this thread's row in chunk ch (main chunks; -1 = none)
  auto entry_of = [&](int ch) __attribute__((always_inline)) {
    int e = -1;
    if (ch < nmc) {
      const int r = ch * CH_ROWS + srow;
      if (r < k) e = idx[(int64_t)q * k + r];
    }
    return e;
  };
  // flat row of this thread's row in chunk ch (-1 = none) from its entry
  auto row_of = [&](int ch, int e) __attribute__((always_inline)) {
    int64_t off = -1;
    if (ch < nmc) {
      if (e >= 0) off = seq * cap + e;
    } else {
      const int r = (ch - nmc) * CH_ROWS + srow;
      if (r < sl) off = seq * T_swa + (sst + r < T_swa ? sst + r : sst + r - T_swa);
    }
    return off;
  };

  // ---- query tile of head group hg (head 16 hg + r16, dims 32 s + 8 qd .. +7)
  f16x8_t a[16];
  f16x8_t alo[2];                 // with RoPE: low terms of steps 14 and 15
  float hinv[4];
  {
    const uint16_t* qp = qv + ((int64_t)q * H_ATT + hg * 16 + r16) * D_LAT + 8 * qd;
    bf16x8_t x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = *(const bf16x8_t*)(qp + 32 * s);
    rope_table<AW_THREADS>(rp, q, rcs);            // while the query bytes are in flight
    float xf[16][8];
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) xf[s][j] = (float)x[s][j];
    if (rp.dims > 0) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2)
          rope_pair(xf[s][2 * p2], xf[s][2 * p2 + 1], 32 * s + 8 * qd + 2 * p2, rp.dims, rcs, 1.f);
    }
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(xf[s][j]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int e = q_exponent(mx);
    const float f = ldexpf(1.f, e);
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[s][j] = (_Float16)(xf[s][j] * f);
    // the rotated query is no longer exact in fp16: its last 64 dims carry a
    // second, low fp16 term (the exact fp32 difference, rounded once)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) alo[s][j] = (_Float16)(xf[14 + s][j] * f - (float)a[14 + s][j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) hinv[j] = ldexpf(1.f, -__shfl(e, 4 * qd + j));
  }
  f32x4_t o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; }

  // ---- pipeline: raw bytes of chunk 0 in flight, entry of chunk 1 in flight
  RawShare<AW_THREADS> raw;
  int64_t cur_off = -1;
  int nxt_e = -1;
  if (nch > 0) {
    cur_off = row_of(0, entry_of(0));
    const bool m0 = 0 < nmc;
    load_share<AW_THREADS>(raw, m0, cur_off >= 0 ? cur_off : (m0 ? seq * cap : seq * T_swa + sst),
                           spart, kv_codes, kv_scales, swa_codes);
    nxt_e = entry_of(1);
  }

  for (int ch = 0; ch < nch; ++ch) {
    const bool is_main = ch < nmc;
    // ---- this chunk's rows, dequantised, into LDS
    {
      const bool valid = cur_off >= 0;
      const float sg = (!is_main && valid) ? swa_scale[cur_off] : 1.f;
      if (tid < CH_ROWS) { rowoff[tid] = cur_off; rowsig[tid] = sg; }
      store_share<AW_THREADS>(raw, is_main, valid, sg, kv[0], kv[1], srow, spart);
    }
    __syncthreads();
    // ---- next chunk's bytes and the entry after it, in flight during the compute
    if (ch + 1 < nch) {
      cur_off = row_of(ch + 1, nxt_e);
      const bool mn = ch + 1 < nmc;
      load_share<AW_THREADS>(raw, mn, cur_off >= 0 ? cur_off : (mn ? seq * cap : seq * T_swa + sst),
                             spart, kv_codes, kv_scales, swa_codes);
      nxt_e = entry_of(ch + 2);
    }

    // ---- S = Q K^T: rows 32*half .. +31 (two 16-row tiles), heads of group hg
    f32x4_t sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = half * 32 + rt * 16 + r16;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = mfma16_f16(a[s], qk_b(kv[0], row, s, qd), acc);
      if (rp.dims > 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mfma16_f16(alo[s], qk_b(kv[0], row, 14 + s, qd), acc);
      }
      const bool valid = rowoff[row] >= 0;
      const float rs = is_main ? 1.f : rowsig[row];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = valid ? acc[j] * hinv[j] * rs : -INFINITY;
      sacc[rt] = acc;
    }

    // ---- online softmax: chunk max per head over both row halves
    float cm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cm[j] = row16_max(fmaxf(sacc[0][j], sacc[1][j]));
    }
    if (r16 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) red_m[half][hg * 16 + 4 * qd + j] = cm[j];
    }
    __syncthreads();
    float alpha[4];
    bool moved = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = hg * 16 + 4 * qd + j;
      // the reference max of a head moves only when a chunk exceeds it by
      // more than AW_LAZY (P then stays below e^AW_LAZY, far inside fp16), so
      // O is rescaled only in the few chunks where some max moved
      const float m_chunk = fmaxf(red_m[0][hh], red_m[1][hh]);
      const float m_new = m_chunk > m_run[j] + AW_LAZY ? m_chunk : m_run[j];
      moved |= m_new != m_run[j];
      float psum = 0.f;
      if (m_new == -INFINITY) {
        alpha[j] = 1.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) pl[hh][half * 32 + rt * 16 + r16] = (_Float16)0.f;
      } else {
        alpha[j] = exp_hw(m_run[j] - m_new);          // 0 when m_run is -inf
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const float p = exp_hw(sacc[rt][j] - m_new); // masked rows: exp(-inf) = 0
          psum += p;
          pl[hh][half * 32 + rt * 16 + r16] = (_Float16)p;
        }
      }
      l_run[j] = l_run[j] * alpha[j] + row16_sum(psum);   // this wave's rows only
      m_run[j] = m_new;
    }
    __syncthreads();

    // ---- O += P V: heads of group hg, dims 256*half .. +255 (16 tiles)
    // (the O rows of this lane are the same heads as its S rows: 16hg + 4qd + j)
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {        // uniform over the wave
#pragma unroll
      for (int t = 0; t < 16; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[t][j] *= alpha[j];
      }
    }
    const _Float16* vrows = is_main ? kv[0] : kv[1];
    const f16x8_t pa0 = *(const f16x8_t*)&pl[hg * 16 + r16][qd * 8];
    const f16x8_t pa1 = *(const f16x8_t*)&pl[hg * 16 + r16][32 + qd * 8];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int n0 = half * 256 + 16 * t;
      o[t] = mfma16_f16(pa0, pv_b(vrows, 0, n0, lane), o[t]);
      o[t] = mfma16_f16(pa1, pv_b(vrows, 32, n0, lane), o[t]);
    }
    __syncthreads();
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
    const int64_t row = ((int64_t)q * H_ATT + hh) * D_LAT + half * 256 + r16;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = o[t][j] * inv;
      const int d = half * 256 + 16 * t + r16;
      if (rp.dims > 0 && half * 256 + 16 * t + 15 >= D_LAT - rp.dims)   // uniform per wave
        v = rope_out_lane(v, d, rp.dims, rcs);
      if (rp.out_bf16) rp.out_bf16[row + 16 * t] = bf16_rne(v);
      else out[row + 16 * t] = v;
    }
    if (lse && half == 0 && r16 == 0)
      lse[(int64_t)q * H_ATT + hh] = L > 0.f ? m_run[j] + logf(L) : -INFINITY;
  }
}

hipError_t launch_attend_wide(const uint16_t* q, const int32_t* q_seq, int Q,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
                              const int32_t* idx, int k, const uint8_t* swa_codes,
                              const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                              const int32_t* swa_len, float* out, float* lse, const RopeArgs& rp,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_attend_wide, dim3((unsigned)Q), dim3(AW_THREADS), 0, stream, q, q_seq,
                     kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale, T_swa, swa_start,
                     swa_len, out, lse, rp);
  return hipGetLastError();
}

}  // namespace csa2
