// Steps a4 / a7: lightning-indexer scores of each query against its visible
// entries (Full layer) or against a candidate pool (Reindex layer).
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3 (indexer Q and K score
// the main-KV entries) and 2.3.2 (Full layers scan the whole causally visible
// range, Reindex layers only the pool); the score form
//   s = sum_h w_h * max(0, q_h . k)       (32 heads x 128)
// follows the mer.dev commentary, section 4.1.
//
// Design: one wave scores 32 entries per step as a 32x32 MFMA tile
// (rows = the query's 32 heads, columns = entries, K = the 128 dims in 8
// bf16 32x32x16 steps).  The query tile stays in registers for the whole
// scan; each lane streams 32 contiguous bytes of one entry's MXFP4 codes
// (its half of the 128 dims) plus the entry's 4 scale bytes, and converts
// them to bf16 with the gfx950 scaled FP4 conversion (exact for the
// power-of-two E8M0 scales).  The ReLU, the
// head weights and the head sum are applied to the accumulator in registers
// and the two lane halves are summed with one cross-lane exchange, so only
// 4 bytes per entry are written.  The next tile's bytes are loaded before
// the current tile's MFMAs issue.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int SC_WAVES = 4;

// TPW: 32-entry tiles per wave; DEPTH: tiles whose bytes are in flight ahead
// of the one being multiplied.
template <bool CAND, int TPW, int DEPTH>
__global__ __launch_bounds__(256) void k_index_score(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const int32_t* __restrict__ q_seq, const int64_t* __restrict__ n_vis,
    const int32_t* __restrict__ cand, int64_t ld_cand, int64_t nchunk, int64_t n_cols,
    const uint8_t* __restrict__ ik_codes, const uint8_t* __restrict__ ik_scales, int64_t cap,
    float* __restrict__ scores, int64_t ld) {
  constexpr int SC_COLS = SC_WAVES * TPW * 32;        // columns per workgroup
  const int q = (int)(blockIdx.x / nchunk);
  const int64_t cbase = (int64_t)(blockIdx.x % nchunk) * SC_COLS;
  const int64_t nv0 = n_vis[q];
  const int64_t nv = nv0 < n_cols ? nv0 : n_cols;     // never past the launch's columns
  if (cbase >= nv) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int64_t seq_base = (int64_t)q_seq[q] * cap;

  // A operand: head r, dims 64*half + 8s .. +7 for step s.
  bf16x8_t a[8];
  const uint16_t* qp = q_idx + ((int64_t)q * H_IDX + r) * D_IDX + half * 64;
#pragma unroll
  for (int s = 0; s < 8; ++s) a[s] = *(const bf16x8_t*)(qp + 8 * s);
  // head weight of each accumulator row this lane holds
  float wr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wr[j] = w[q * H_IDX + 8 * (j >> 2) + 4 * half + (j & 3)];

  const int32_t* crow = CAND ? cand + (int64_t)q * ld_cand : nullptr;
  float* srow = scores + (int64_t)q * ld;

  auto load = [&](int64_t col0, u32x4_t& c0, u32x4_t& c1, uint32_t& scw) {
    const int64_t c = col0 + r;
    const int64_t cc = c < nv ? c : col0;
    const int64_t e = CAND ? (int64_t)crow[cc] : cc;
    const uint8_t* cp = ik_codes + (seq_base + e) * 64 + half * 32;
    c0 = *(const u32x4_t*)cp;
    c1 = *(const u32x4_t*)(cp + 16);
    scw = *(const uint32_t*)(ik_scales + (seq_base + e) * 4);
  };

  // ring of DEPTH + 1 tiles: slot t % (DEPTH + 1) holds tile t
  u32x4_t r0[DEPTH + 1], r1[DEPTH + 1];
  uint32_t rs[DEPTH + 1];
  const int64_t step = SC_WAVES * 32;
  const int64_t col_first = cbase + (int64_t)wave * 32;
#pragma unroll
  for (int t = 0; t < DEPTH; ++t) {
    const int64_t c0 = col_first + t * step;
    if (t < TPW && c0 < nv) load(c0, r0[t], r1[t], rs[t]);
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t col0 = col_first + t * step;
    if (col0 >= nv) break;
    {
      const int tn = t + DEPTH;
      const int64_t cn = col_first + tn * step;
      if (tn < TPW && cn < nv) load(cn, r0[tn % (DEPTH + 1)], r1[tn % (DEPTH + 1)], rs[tn % (DEPTH + 1)]);
    }
    const int sl = t % (DEPTH + 1);
    const u32x4_t c0 = r0[sl], c1 = r1[sl];
    const uint32_t scw = rs[sl];
    const float s_lo = e8m0_val((scw >> (16 * half)) & 0xFFu);
    const float s_hi = e8m0_val((scw >> (16 * half + 8)) & 0xFFu);
    f32x16_t acc = {};
    acc = mfma32_bf16(a[0], fp4x8_to_bf16_pow2(c0[0], s_lo), acc);
    acc = mfma32_bf16(a[1], fp4x8_to_bf16_pow2(c0[1], s_lo), acc);
    acc = mfma32_bf16(a[2], fp4x8_to_bf16_pow2(c0[2], s_lo), acc);
    acc = mfma32_bf16(a[3], fp4x8_to_bf16_pow2(c0[3], s_lo), acc);
    acc = mfma32_bf16(a[4], fp4x8_to_bf16_pow2(c1[0], s_hi), acc);
    acc = mfma32_bf16(a[5], fp4x8_to_bf16_pow2(c1[1], s_hi), acc);
    acc = mfma32_bf16(a[6], fp4x8_to_bf16_pow2(c1[2], s_hi), acc);
    acc = mfma32_bf16(a[7], fp4x8_to_bf16_pow2(c1[3], s_hi), acc);
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) part += wr[j] * relu_f32(acc[j]);
    part += __shfl_xor(part, 32);
    const int64_t c = col0 + r;
    if (half == 0 && c < nv) srow[c] = part;
  }
}

template <bool CAND, int TPW, int DEPTH>
static void launch_variant(dim3 grid, hipStream_t stream, const uint16_t* q_idx, const float* w,
                           const int32_t* q_seq, const int64_t* n_vis, const int32_t* cand,
                           int64_t ld_cand, int64_t nchunk, int64_t n_cols,
                           const uint8_t* ik_codes, const uint8_t* ik_scales, int64_t cap,
                           float* scores, int64_t ld) {
  hipLaunchKernelGGL((k_index_score<CAND, TPW, DEPTH>), grid, dim3(256), 0, stream, q_idx, w,
                     q_seq, n_vis, cand, ld_cand, nchunk, n_cols, ik_codes, ik_scales, cap, scores,
                     ld);
}

hipError_t launch_index_score(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                              const int64_t* n_vis, const int32_t* cand, int64_t ld_cand, int Q,
                              int64_t n_cols, const uint8_t* ik_codes, const uint8_t* ik_scales,
                              int64_t cap, float* scores, int64_t ld, hipStream_t stream) {
  // Tiles per wave: the largest of 32, 16, 8, 2, 1 that still launches at
  // least 1024 workgroups (4 per CU); long scans keep two tiles in flight.
  // (Swept on MI355X: 1M-entry scans want 32 tiles x 2 in flight, 64K-entry
  // scans 8-16, 16K-entry Reindex pools 1-2.)
  int tpw = 1;
  for (int t : {32, 16, 8, 2}) {
    const int64_t wgs = (int64_t)Q * ((n_cols + 128 * t - 1) / (128 * t));
    if (wgs >= 1024) { tpw = t; break; }
  }
  const int64_t cols = (int64_t)SC_WAVES * tpw * 32;
  const int64_t nchunk = (n_cols + cols - 1) / cols;
  const dim3 grid((unsigned)(nchunk * Q));
#define CSA2_SCORE_CASE(T, D)                                                                       \
  case T:                                                                                          \
    if (cand) launch_variant<true, T, D>(grid, stream, q_idx, w, q_seq, n_vis, cand, ld_cand,      \
                                         nchunk, n_cols, ik_codes, ik_scales, cap, scores, ld);    \
    else launch_variant<false, T, D>(grid, stream, q_idx, w, q_seq, n_vis, cand, ld_cand, nchunk,  \
                                     n_cols, ik_codes, ik_scales, cap, scores, ld);                \
    break;
  switch (tpw) {
    CSA2_SCORE_CASE(32, 2)
    CSA2_SCORE_CASE(16, 2)
    CSA2_SCORE_CASE(8, 2)
    CSA2_SCORE_CASE(2, 1)
    default:
    CSA2_SCORE_CASE(1, 1)
  }
#undef CSA2_SCORE_CASE
  return hipGetLastError();
}

}  // namespace csa2
