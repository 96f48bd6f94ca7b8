// Steps a8 + a9: gather the selected FP4 main-KV rows and the FP8 SWA rows
// of each query and run 64-head attention over them with the latent used as
// both key and value, with an online softmax.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: every query attends to
// its selected main-KV entries together with the layer's sliding-window KV;
// the 512-d latent is shared by the heads (MLA style) and is both key and
// value; section 2.4.4: main KV is dequantised from FP4 before attention,
// SWA KV stays FP8.
//
// Design.  A workgroup of 256 threads owns (query, 16 heads, a run of
// 64-row chunks).  Main-KV chunks and SWA chunks are separate, so every
// chunk has one row type and the MFMAs stay in uniform control flow.
//   query     the 16 heads' rows are converted once to fp16 in LDS, each
//             head scaled by a power of two (undone on the scores).
//   staging   thread t loads the (t & 63)-th row's quarter t >> 6 straight
//             from HBM (its own idx lookup, no barrier in between) and
//             writes it dequantised to fp16 in LDS (see attend_stage.h).
//   S = Q K^T 16 heads x 64 rows, 16x16x32 fp16 MFMA, wave w rows 16w..+15.
//   softmax   running max / sum per head, reductions through LDS.
//   O += P V  16 heads x 512 dims, 16x16x32 fp16 MFMA, wave w dims
//             128w..+127; V columns come from the staged rows through
//             transposing LDS reads.
// Decode (few queries) splits the chunks of a query over several
// workgroups and merges the partial (max, sum, O) by log-sum-exp in a second
// kernel (merging in the last workgroup to finish needs an agent-scope fence,
// which writes back the whole L2 of its XCD on MI355X and measured 4x slower).
#include "common.h"
#include "launch.h"
#include "attend_stage.h"

namespace csa2 {

constexpr int AT_HG = 16;          // heads per workgroup
constexpr int AT_PAD = 8;          // fp16 padding of an LDS row
constexpr int AT_MAX_SWA = 128;
constexpr int AT_TARGET_WG = 1024; // workgroups a decode launch aims for
constexpr int AT_WIDE_MIN_Q = 256;  // from this many queries on, one workgroup per query

__global__ __launch_bounds__(256, 1) void k_attend(
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa_codes,
    const float* __restrict__ swa_scale, int64_t T_swa, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml, int nsplit, int cps, RopeArgs rp) {
  __shared__ __align__(16) _Float16 kv[2][CH_ROWS * KV_LD];         // K (+ V of main rows), V of SWA rows
  __shared__ __align__(16) _Float16 qs[AT_HG][D_LAT + AT_PAD];     // fp16 query rows
  __shared__ __align__(16) _Float16 pl[AT_HG][CH_ROWS + AT_PAD];   // P of the chunk
  __shared__ float red_m[4][AT_HG], red_l[4][AT_HG];
  __shared__ int64_t rowoff[CH_ROWS];                               // entry / SWA row, -1 = none
  __shared__ float rowsig[CH_ROWS];
  __shared__ float qinv[AT_HG];                                     // 2^-e of each head
  __shared__ f32x2_t rcs[ROPE_MAX_PAIRS];                           // RoPE (cos, sin) per pair
  __shared__ __align__(16) _Float16 qs_lo[AT_HG][ROPE_MAX_DIMS + AT_PAD];  // low fp16 terms, last 64 dims

  const int sp = blockIdx.x % nsplit;
  const int hq = blockIdx.x / nsplit;
  const int hg = hq & 3, q = hq >> 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, qd = lane >> 4;
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  const int ch_beg = sp * cps;
  // The first chunk's selected id (when it is a main-KV chunk) and the query
  // rows go out before the query's sequence and window arrive: neither
  // depends on them.
  int id0 = -1;
  if (ch_beg < nmc) {
    const int r0 = ch_beg * CH_ROWS + (tid & 63);
    id0 = idx[(int64_t)q * k + (r0 < k ? r0 : k - 1)];
  }
  const int qh = tid >> 4, qpart = tid & 15;     // query conversion: head, 32-dim part
  bf16x8_t x[4];
  {
    const bf16x8_t* qp = (const bf16x8_t*)(qv + ((int64_t)q * H_ATT + hg * AT_HG + qh) * D_LAT +
                                           qpart * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = qp[i];
  }
  const int64_t seq = q_seq[q];
  const int64_t sst = swa_start[q];
  int64_t sl64 = swa_len[q];
  if (sst < 0 || sst >= T_swa) sl64 = 0;                     // ring: start must be a slot
  else if (sl64 > T_swa) sl64 = T_swa;                       // at most one lap
  const int sl = sl64 < 0 ? 0 : (sl64 > AT_MAX_SWA ? AT_MAX_SWA : (int)sl64);
  const int nch = nmc + (sl + CH_ROWS - 1) / CH_ROWS;
  const int ch_end = min(ch_beg + cps, nch);

  // This thread's staging row (row t & 63 of chunk ch) in two steps: row_req
  // issues the load its row depends on (the selected id, or the SWA row's
  // scale), clamped into range, and row_res turns it into the flat row
  // (-1 = none) and the row scale, so other loads can be issued in between.
  struct RowReq { int e; float s; };
  auto row_req = [&](int ch) __attribute__((always_inline)) {
    RowReq rq{-1, 1.f};
    const bool main_ch = ch < nmc;             // uniform
    const int r = (main_ch ? ch * CH_ROWS : (ch - nmc) * CH_ROWS) + (tid & 63);
    if (main_ch) {
      rq.e = idx[(int64_t)q * k + (r < k ? r : k - 1)];
    } else {
      const int rr = r < sl ? r : sl - 1;       // an SWA chunk exists only when sl >= 1
      rq.s = swa_scale[seq * T_swa + (sst + rr < T_swa ? sst + rr : sst + rr - T_swa)];
    }
    return rq;
  };
  auto row_res = [&](int ch, const RowReq& rq, float& sg) __attribute__((always_inline)) {
    const bool main_ch = ch < nmc;
    const int r = (main_ch ? ch * CH_ROWS : (ch - nmc) * CH_ROWS) + (tid & 63);
    int64_t off = -1;
    sg = 1.f;
    if (main_ch) {
      if (r < k && rq.e >= 0) off = seq * cap + rq.e;
    } else if (r < sl) {
      off = seq * T_swa + (sst + r < T_swa ? sst + r : sst + r - T_swa);
      sg = rq.s;
    }
    return off;
  };
  auto row_of = [&](int ch, float& sg) __attribute__((always_inline)) {
    return row_res(ch, row_req(ch), sg);
  };
  // a readable row of chunk ch in place of a missing one
  auto readable = [&](int64_t off, bool main_ch) __attribute__((always_inline)) {
    return off >= 0 ? off : (main_ch ? seq * cap : seq * T_swa + sst);
  };
  // the first chunk's row id, then its raw bytes, are in flight before the
  // query work
  const RowReq rq0 = ch_beg < nmc ? RowReq{id0, 1.f} : row_req(ch_beg < ch_end ? ch_beg : 0);
  float nsg = 1.f;
  int64_t noff = -1;
  RawShare<256> raw;

  // ---- query: thread t converts head t >> 4, dims 32 (t & 15) .. +31
  {
    const int hh = qh, part = qpart;
    // keep the wait for the row id below the query loads (the scheduler
    // would otherwise move the loads after it)
    __builtin_amdgcn_sched_barrier(0);
    if (ch_beg < ch_end) {
      noff = row_res(ch_beg, rq0, nsg);
      load_share<256>(raw, ch_beg < nmc, readable(noff, ch_beg < nmc), tid >> 6, kv_codes, kv_scales,
                      swa_codes);
    }
    rope_table<256>(rp, q, rcs);                   // while the query bytes are in flight
    float xf[32];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) xf[8 * i + j] = (float)x[i][j];
#pragma unroll
    for (int p2 = 0; p2 < 16; ++p2)
      rope_pair(xf[2 * p2], xf[2 * p2 + 1], part * 32 + 2 * p2, rp.dims, rcs, 1.f);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(xf[i]));
    mx = row16_max(mx);                          // the 16 threads of head hh
    const int e = q_exponent(mx);
    const float f = ldexpf(1.f, e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x8_t y, ylo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = xf[8 * i + j] * f;
        y[j] = (_Float16)v;
        ylo[j] = (_Float16)(v - (float)y[j]);          // exact difference, rounded once
      }
      *(f16x8_t*)&qs[hh][part * 32 + 8 * i] = y;
      if (rp.dims > 0 && part >= 14) *(f16x8_t*)&qs_lo[hh][(part - 14) * 32 + 8 * i] = ylo;
    }
    if (part == 0) qinv[hh] = ldexpf(1.f, -e);
  }

  f16x8_t a[16];                  // query tile: head r16, dims 32 s + 8 qd .. +7 for step s
  f16x8_t alo[2];                 // with RoPE: low terms of steps 14 and 15
  f32x4_t o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4], hinv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; }

  for (int ch = ch_beg; ch < ch_end; ++ch) {
    const bool is_main = ch < nmc;                 // uniform over the workgroup
    // ---- stage: thread t takes row t & 63, quarter t >> 6
    {
      float sg = nsg;
      const int64_t off = ch == ch_beg ? noff : row_of(ch, sg);
      const bool valid = off >= 0;
      if (ch != ch_beg)
        load_share<256>(raw, is_main, readable(off, is_main), tid >> 6, kv_codes, kv_scales,
                        swa_codes);
      if (tid < CH_ROWS) { rowoff[tid] = off; rowsig[tid] = sg; }
      store_share<256>(raw, is_main, valid, sg, kv[0], kv[1], tid & 63, tid >> 6);
    }
    __syncthreads();
    if (ch == ch_beg) {
#pragma unroll
      for (int s = 0; s < 16; ++s) a[s] = *(const f16x8_t*)&qs[r16][32 * s + 8 * qd];
      if (rp.dims > 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) alo[s] = *(const f16x8_t*)&qs_lo[r16][32 * s + 8 * qd];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) hinv[j] = qinv[4 * qd + j];
    }

    // ---- S = Q K^T for rows 16*wave .. +15 (lane column r16)
    const int lr = wave * 16 + r16;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) sacc = mfma16_f16(a[s], qk_b(kv[0], lr, s, qd), sacc);
    if (rp.dims > 0) {                             // the rotated query's low terms
#pragma unroll
      for (int s = 0; s < 2; ++s) sacc = mfma16_f16(alo[s], qk_b(kv[0], lr, 14 + s, qd), sacc);
    }
    const bool valid = rowoff[lr] >= 0;
    const float rs = is_main ? 1.f : rowsig[lr];
#pragma unroll
    for (int j = 0; j < 4; ++j) sacc[j] = valid ? sacc[j] * hinv[j] * rs : -INFINITY;

    // ---- online softmax over this chunk
    float cm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cm[j] = row16_max(sacc[j]);      // over the 16 rows of the wave
    if (r16 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) red_m[wave][4 * qd + j] = cm[j];
    }
    __syncthreads();
    float alpha[4], p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 4 * qd + j;
      const float cmax = fmaxf(fmaxf(red_m[0][hh], red_m[1][hh]), fmaxf(red_m[2][hh], red_m[3][hh]));
      const float m_new = fmaxf(m_run[j], cmax);
      if (m_new == -INFINITY) {
        alpha[j] = 1.f;
        p[j] = 0.f;
      } else {
        alpha[j] = exp_hw(m_run[j] - m_new);            // 0 when m_run is -inf
        p[j] = valid ? exp_hw(sacc[j] - m_new) : 0.f;
      }
      m_run[j] = m_new;
      pl[hh][lr] = (_Float16)p[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = row16_sum(p[j]);
      if (r16 == 0) red_l[wave][4 * qd + j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 4 * qd + j;
      l_run[j] = l_run[j] * alpha[j] + ((red_l[0][hh] + red_l[1][hh]) + (red_l[2][hh] + red_l[3][hh]));
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t][j] *= alpha[j];
    }

    // ---- O += P V for dims 128*wave .. +127
    const _Float16* vrows = is_main ? kv[0] : kv[1];
    const f16x8_t pa0 = *(const f16x8_t*)&pl[r16][qd * 8];
    const f16x8_t pa1 = *(const f16x8_t*)&pl[r16][32 + qd * 8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int n0 = wave * 128 + 16 * t;
      o[t] = mfma16_f16(pa0, pv_b(vrows, 0, n0, lane), o[t]);
      o[t] = mfma16_f16(pa1, pv_b(vrows, 32, n0, lane), o[t]);
    }
    __syncthreads();
  }

  // ---- write the result (single split) or the partial state
  const int head0 = hg * AT_HG + 4 * qd;
  if (nsplit == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float inv = l_run[j] > 0.f ? 1.f / l_run[j] : 0.f;
      const int64_t row = ((int64_t)q * H_ATT + head0 + j) * D_LAT + wave * 128 + r16;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float v = o[t][j] * inv;
        const int d = wave * 128 + 16 * t + r16;
        if (rp.dims > 0 && wave * 128 + 16 * t + 15 >= D_LAT - rp.dims)   // uniform per wave
          v = rope_out_lane(v, d, rp.dims, rcs);
        if (rp.out_bf16) rp.out_bf16[row + 16 * t] = bf16_rne(v);
        else out[row + 16 * t] = v;
      }
      if (lse && wave == 0 && r16 == 0)
        lse[(int64_t)q * H_ATT + head0 + j] = l_run[j] > 0.f ? m_run[j] + logf(l_run[j]) : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t slot = ((int64_t)q * nsplit + sp) * H_ATT + head0 + j;
    float* op = part_o + slot * D_LAT + wave * 128 + r16;
#pragma unroll
    for (int t = 0; t < 8; ++t) op[16 * t] = o[t][j];
    if (wave == 0 && r16 == 0) {
      part_ml[2 * slot] = m_run[j];
      part_ml[2 * slot + 1] = l_run[j];
    }
  }
}

// Merge the per-split partial states of one (query, head) by log-sum-exp.
// Every split wrote its state (an empty split: max -inf, sum 0, O = 0).  A
// thread owns 4 dims; it loads the states of 16 splits at a time, all
// loads in flight together (indices past the last split re-read the last
// one with weight 0), then folds them into a running (max, sum, O).
constexpr int AT_MAX_SPLITS = 64;
constexpr int AT_MERGE_BATCH = 16;

__global__ __launch_bounds__(128) void k_attend_combine(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        int nsplit, float* __restrict__ out,
                                                        float* __restrict__ lse, RopeArgs rp) {
  const int qh = blockIdx.x;              // q * 64 + head
  const int q = qh / H_ATT, h = qh % H_ATT;
  const int d0 = threadIdx.x * 4;
  const int64_t slot0 = (int64_t)q * nsplit * H_ATT + h;    // split s: slot0 + s * H_ATT
  const int64_t pos = rp.dims > 0 ? rp.q_pos[q] : 0;        // in flight with the partials
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += AT_MERGE_BATCH) {
    f32x2_t ml[AT_MERGE_BATCH];
    f32x4_t ov[AT_MERGE_BATCH];
#pragma unroll
    for (int i = 0; i < AT_MERGE_BATCH; ++i) {
      const int si = s0 + i < nsplit ? s0 + i : nsplit - 1;
      const int64_t slot = slot0 + (int64_t)si * H_ATT;
      ml[i] = *(const f32x2_t*)(part_ml + 2 * slot);
      ov[i] = *(const f32x4_t*)(part_o + slot * D_LAT + d0);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < AT_MERGE_BATCH; ++i)
      if (s0 + i < nsplit && ml[i][1] > 0.f) bm = fmaxf(bm, ml[i][0]);
    const float nM = fmaxf(M, bm);
    if (nM == -INFINITY) continue;                      // nothing attended so far
    const float sc = exp_hw(M - nM);                      // 0 while M is -inf
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < AT_MERGE_BATCH; ++i) {
      const float w = (s0 + i < nsplit && ml[i][1] > 0.f) ? exp_hw(ml[i][0] - nM) : 0.f;
      L += ml[i][1] * w;
      acc += ov[i] * w;
    }
    M = nM;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4_t v = acc * inv;
  if (rp.dims > 0 && d0 + 3 >= D_LAT - rp.dims) {
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const int d = d0 + 2 * p2, base = D_LAT - rp.dims;
      if (d >= base) {
        const f32x2_t cs = rope_cs(pos, (d - base) >> 1, rp);
        const float a = v[2 * p2], b = v[2 * p2 + 1];
        v[2 * p2] = a * cs[0] + b * cs[1];               // turned back by the query's angle
        v[2 * p2 + 1] = b * cs[0] - a * cs[1];
      }
    }
  }
  if (rp.out_bf16) {
    const uint32_t lo = (uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16);
    const uint32_t hi = (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16);
    *(uint2*)(rp.out_bf16 + (int64_t)qh * D_LAT + d0) = make_uint2(lo, hi);
  } else {
    *(f32x4_t*)(out + (int64_t)qh * D_LAT + d0) = v;
  }
  if (lse && threadIdx.x == 0) lse[qh] = L > 0.f ? M + logf(L) : -INFINITY;
}

// ------------------------------------------------------------ host side
static void attend_plan(int Q, int k, int& nsplit, int& cps) {
  const int nch = (k + CH_ROWS - 1) / CH_ROWS + AT_MAX_SWA / CH_ROWS;
  const int groups = Q * (H_ATT / AT_HG);
  int want = (AT_TARGET_WG + groups - 1) / groups;
  if (want < 1) want = 1;
  cps = (nch + want - 1) / want;
  if (cps < 1) cps = 1;
  nsplit = (nch + cps - 1) / cps;
  while (nsplit > AT_MAX_SPLITS) { ++cps; nsplit = (nch + cps - 1) / cps; }
  if (nsplit < 1) nsplit = 1;
}

// workspace: [partial O: Q * nsplit * 64 * 512 fp32][partial (max, sum)]
static size_t attend_ws_for(int Q, int nsplit) {
  if (nsplit <= 1) return 0;
  return (size_t)Q * nsplit * H_ATT * (D_LAT + 2) * sizeof(float);
}

size_t attend_ws_bytes(int Q, int k) {
  if (Q >= AT_WIDE_MIN_Q) return 0;
  int nsplit, cps;
  attend_plan(Q, k, nsplit, cps);
  return attend_ws_for(Q, nsplit);
}

hipError_t launch_attend(const uint16_t* q, const int32_t* q_seq, int Q, const uint8_t* kv_codes,
                         const uint8_t* kv_scales, int64_t cap, const int32_t* idx, int k,
                         const uint8_t* swa_codes, const float* swa_scale, int64_t T_swa,
                         const int64_t* swa_start, const int32_t* swa_len, float* out, float* lse,
                         void* ws, size_t ws_bytes, const RopeArgs& rp, hipStream_t stream) {
  // many queries (prefill): one workgroup per query over all heads
  if (Q >= AT_WIDE_MIN_Q)
    return launch_attend_wide(q, q_seq, Q, kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale,
                              T_swa, swa_start, swa_len, out, lse, rp, stream);
  int nsplit, cps;
  attend_plan(Q, k, nsplit, cps);
  const int nch = (k + CH_ROWS - 1) / CH_ROWS + AT_MAX_SWA / CH_ROWS;
  while (nsplit > 1 && (ws == nullptr || attend_ws_for(Q, nsplit) > ws_bytes)) {
    ++cps;                                   // fewer, longer splits until the partials fit
    nsplit = (nch + cps - 1) / cps;
  }
  if (nsplit <= 1) { nsplit = 1; cps = nch; }
  float* part_o = (float*)ws;
  float* part_ml = nsplit > 1 ? part_o + (size_t)Q * nsplit * H_ATT * D_LAT : nullptr;
  hipLaunchKernelGGL(k_attend, dim3((unsigned)(Q * (H_ATT / AT_HG) * nsplit)), dim3(256), 0,
                     stream, q, q_seq, kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale,
                     T_swa, swa_start, swa_len, out, lse, part_o, part_ml, nsplit, cps, rp);
  if (nsplit > 1)
    hipLaunchKernelGGL(k_attend_combine, dim3((unsigned)(Q * H_ATT)), dim3(128), 0, stream,
                       (const float*)part_o, (const float*)part_ml, nsplit, out, lse, rp);
  return hipGetLastError();
}

}  // namespace csa2
