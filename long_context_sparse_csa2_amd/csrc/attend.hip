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
#include "select_core.h"

namespace csa2 {

constexpr int AT_HG = 16;          // heads per workgroup
constexpr int AT_PAD = 8;          // fp16 padding of an LDS row
constexpr int AT_MAX_SWA = 128;
constexpr int AT_WIDE_MIN_Q = 256;  // from this many queries on, one workgroup per query

// LDS of one 256-thread attention workgroup, except the SWA rows' scaled V
// copy (kv1), which the fused selection kernel overlays on its selection
// state.
struct AttendLds {
  alignas(16) _Float16 kv[CH_ROWS * KV_LD];             // K (and V of main rows) of the chunk
  alignas(16) _Float16 qs[AT_HG][D_LAT + AT_PAD];       // fp16 query rows
  alignas(16) _Float16 pl[AT_HG][CH_ROWS + AT_PAD];     // P of the chunk
  float red_m[4][AT_HG], red_l[4][AT_HG];
  int64_t rowoff[CH_ROWS];                               // entry / SWA row, -1 = none
  float rowsig[CH_ROWS];
  float qinv[AT_HG];                                     // 2^-e of each head
  f32x2_t rcs[ROPE_MAX_PAIRS];                           // RoPE (cos, sin) per pair
  alignas(16) _Float16 qs_lo[AT_HG][ROPE_MAX_DIMS + AT_PAD];  // low fp16 terms, last 64 dims
};

// A query's sequence and SWA window (ring start, length clamped to one lap
// and to AT_MAX_SWA rows; a start outside the ring gives no rows).
struct AttendQuery {
  int64_t seq, sst;
  int sl;
};

__device__ __forceinline__ AttendQuery attend_query(int q, const int32_t* __restrict__ q_seq,
                                                    const int64_t* __restrict__ swa_start,
                                                    const int32_t* __restrict__ swa_len,
                                                    int64_t T_swa) {
  AttendQuery a;
  a.seq = q_seq[q];
  a.sst = swa_start[q];
  int64_t sl64 = swa_len[q];
  if (a.sst < 0 || a.sst >= T_swa) sl64 = 0;                 // ring: start must be a slot
  else if (sl64 > T_swa) sl64 = T_swa;                       // at most one lap
  a.sl = sl64 < 0 ? 0 : (sl64 > AT_MAX_SWA ? AT_MAX_SWA : (int)sl64);
  return a;
}

// This thread's share of the query rows of head group hg: head tid >> 4,
// dims 32 (tid & 15) .. +31 (threads 0..255).
__device__ __forceinline__ void attend_query_rows(bf16x8_t (&x)[4], const uint16_t* __restrict__ qv,
                                                  int q, int hg) {
  const int tid = threadIdx.x;
  const bf16x8_t* qp = (const bf16x8_t*)(qv + ((int64_t)q * H_ATT + hg * AT_HG + (tid >> 4)) * D_LAT +
                                         (tid & 15) * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = qp[i];
}

// Workgroup b -> (unit, head group): the four head-group workgroups of one
// unit (query, split) get indices 8 apart, so the round-robin dispatch over
// the 8 XCDs puts them on one XCD and its L2 serves the rows all four
// gather.  A launch has ceil(units / 8) * 32 workgroups; those past the
// last unit return at once.
__device__ __forceinline__ void unit_of(int b, int& u, int& hg) {
  u = (b >> 5) * 8 + (b & 7);
  hg = (b >> 3) & 3;
}
static inline unsigned unit_grid(int units) { return (unsigned)((units + 7) / 8 * 32); }

// One workgroup's part of a query's attention: head group hg (16 heads),
// chunks sp * cps .. of the query's main-KV chunks followed by its SWA
// chunks; id_of(r) is the selected entry of main row r (r < k); id0 that of
// this thread's row of the first chunk (when it is a main chunk), requested
// by the caller before the query rows x and the scalars aq.  Writes the
// final output when nsplit == 1, else the partial (max, sum, O) state; NT:
// through nontemporal stores (the merge kernel reads them from another
// XCD, so keeping them in this XCD's L2 gains nothing: measured on MI355X,
// the 8-sequence decode step with five Reuse layers 2.4 % faster; the fused
// selection kernel measured no faster with them and keeps plain stores).
template <bool NT = false, typename IdOf>
__device__ __forceinline__ void attend_body(
    int q, int hg, int sp, int nsplit, int cps, IdOf id_of, int id0, const bf16x8_t (&x)[4],
    const AttendQuery& aq, const uint8_t* __restrict__ kv_codes,
    const uint8_t* __restrict__ kv_scales, int64_t cap, int k,
    const uint8_t* __restrict__ swa_codes, const float* __restrict__ swa_scale, int64_t T_swa,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, const RopeArgs& rp, AttendLds& L, _Float16* kv1) {
  _Float16* const kv0 = L.kv;
  auto& qs = L.qs;
  auto& pl = L.pl;
  auto& red_m = L.red_m;
  auto& red_l = L.red_l;
  auto& rowoff = L.rowoff;
  auto& rowsig = L.rowsig;
  auto& qinv = L.qinv;
  auto& rcs = L.rcs;
  auto& qs_lo = L.qs_lo;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: scalar registers
  const int r16 = lane & 15, qd = lane >> 4;
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  const int ch_beg = sp * cps;
  const int qh = tid >> 4, qpart = tid & 15;     // query conversion: head, 32-dim part
  const int64_t seq = aq.seq, sst = aq.sst;
  const int sl = aq.sl;
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
      rq.e = id_of(r < k ? r : k - 1);
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
      load_share<256>(raw, ch_beg < nmc, readable(noff, ch_beg < nmc), wave, kv_codes, kv_scales,
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
    // ---- stage: thread t takes row t & 63, quarter t >> 6.  The chunk's
    // raw bytes (row noff, scale nsg) are in flight in `raw`; once they are
    // in LDS the next chunk's row id and then its bytes are requested into
    // the same registers, so they arrive during this chunk's MFMAs.
    {
      const bool more = ch + 1 < ch_end;          // uniform
      RowReq rqn{-1, 1.f};
      if (more) rqn = row_req(ch + 1);
      const int64_t off = noff;
      const float sg = nsg;
      if (tid < CH_ROWS) { rowoff[tid] = off; rowsig[tid] = sg; }
      store_share<256>(raw, is_main, off >= 0, sg, kv0, kv1, tid & 63, wave);
      if (more) {
        const bool nmain = ch + 1 < nmc;
        noff = row_res(ch + 1, rqn, nsg);
        load_share<256>(raw, nmain, readable(noff, nmain), wave, kv_codes, kv_scales,
                        swa_codes);
      }
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
    for (int s = 0; s < 16; ++s) sacc = mfma16_f16(a[s], qk_b(kv0, lr, s, qd), sacc);
    if (rp.dims > 0) {                             // the rotated query's low terms
#pragma unroll
      for (int s = 0; s < 2; ++s) sacc = mfma16_f16(alo[s], qk_b(kv0, lr, 14 + s, qd), sacc);
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
    const _Float16* vrows = is_main ? kv0 : kv1;
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
    for (int t = 0; t < 8; ++t) {
      if constexpr (NT) __builtin_nontemporal_store(o[t][j], op + 16 * t);
      else op[16 * t] = o[t][j];
    }
    if (wave == 0 && r16 == 0) {
      if constexpr (NT) {
        __builtin_nontemporal_store(m_run[j], part_ml + 2 * slot);
        __builtin_nontemporal_store(l_run[j], part_ml + 2 * slot + 1);
      } else {
        part_ml[2 * slot] = m_run[j];
        part_ml[2 * slot + 1] = l_run[j];
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_attend(
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa_codes,
    const float* __restrict__ swa_scale, int64_t T_swa, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml, int nsplit, int cps, int Q,
    RopeArgs rp) {
  __shared__ AttendLds L;
  __shared__ __align__(16) _Float16 kv1[CH_ROWS * KV_LD];          // V of SWA rows
  int u, hg;
  unit_of(blockIdx.x, u, hg);
  if (u >= Q * nsplit) return;
  const int q = u / nsplit, sp = u % nsplit;
  const int tid = threadIdx.x;
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  // The first chunk's selected id (when it is a main-KV chunk) and the query
  // rows go out before the query's sequence and window arrive: neither
  // depends on them.
  const int32_t* irow = idx + (int64_t)q * k;
  int id0 = -1;
  if (sp * cps < nmc) {
    const int r0 = sp * cps * CH_ROWS + (tid & 63);
    id0 = irow[r0 < k ? r0 : k - 1];
  }
  bf16x8_t x[4];
  attend_query_rows(x, qv, q, hg);
  const AttendQuery aq = attend_query(q, q_seq, swa_start, swa_len, T_swa);
  attend_body<true>(q, hg, sp, nsplit, cps, [&](int r) __attribute__((always_inline)) { return irow[r]; },
              id0, x, aq, kv_codes, kv_scales, cap, k, swa_codes, swa_scale, T_swa, out, lse,
              part_o, part_ml, rp, L, kv1);
}

// Merge the per-split partial states of one (query, head) by log-sum-exp.
// Every split wrote its state (an empty split: max -inf, sum 0, O = 0).  A
// thread owns 4 dims; it loads the states of up to 16 splits at a time,
// all loads in flight together (slots past the last split are not read:
// re-reading the last split there cost the 4 x 2^20 decode step 4 %), then
// folds them into a running (max, sum, O).
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
      const int64_t slot = slot0 + (int64_t)(s0 + i) * H_ATT;
      ml[i] = f32x2_t{-INFINITY, 0.f};
      ov[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // only the splits that exist (no clamped re-reads of the last one);
      // the partial rows with the nontemporal policy: each is read once
      if (s0 + i < nsplit) {
        ml[i] = *(const f32x2_t*)(part_ml + 2 * slot);
        ov[i] = __builtin_nontemporal_load((const f32x4_t*)(part_o + slot * D_LAT + d0));
      }
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


// ------------------------------------------------------------ fused
// Selection and attention in one kernel (decode): every main-chunk
// workgroup of a query runs the query's whole selection itself (the
// selection is deterministic, so they all agree), keeps the entries of its
// own rows (cps consecutive 64-row chunks: more than one when one chunk per
// workgroup would not fit the device's CUs in one round) and attends over
// them; the workgroup of head group 0 and split 0 also writes the selection
// out.  This removes the kernel boundary and the round trip of the ids
// through memory between the two steps (cross-workgroup hand-offs inside a
// kernel measured slower on MI355X than a kernel boundary).  Workgroups
// whose chunks are all SWA chunks skip the selection.  512 threads: the
// selection runs on all eight waves, the attention on the first four (the
// other four end after the selection; a barrier waits only for the waves
// that have not ended).
constexpr int SA_NT = 512;
constexpr int SA_MAX_CPS = 8;                   // a thread per row id of the workgroup's chunks
static_assert(SA_MAX_CPS * CH_ROWS <= SA_NT, "one thread per kept row id");

template <int MODE>
__global__ __launch_bounds__(SA_NT, 1) void k_select_attend(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, LevelDesc d,
    const uint32_t* __restrict__ lv, int kk, int k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ pool, int64_t* __restrict__ pool_len, int vec_out, int spec,
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const uint8_t* __restrict__ swa_codes, const float* __restrict__ swa_scale, int64_t T_swa,
    const int64_t* __restrict__ swa_start, const int32_t* __restrict__ swa_len,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int nsplit, int cps, int Q) {
  __shared__ AttendLds L;
  __shared__ union alignas(16) SaOverlay {
    SelShared<SA_NT> sel;                       // main chunks: the selection state
    _Float16 kv1[CH_ROWS * KV_LD];              // SWA chunks: V of the SWA rows
  } U;
  __shared__ int32_t cid[SA_MAX_CPS * CH_ROWS];  // entries of this workgroup's rows
  int u, hg;
  unit_of(blockIdx.x, u, hg);
  if (u >= Q * nsplit) return;
  const int q = u / nsplit, sp = u % nsplit;
  const int tid = threadIdx.x;
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  const int row0 = sp * cps * CH_ROWS;          // first row of the workgroup's chunks
  const bool main_ch = sp * cps < nmc;          // uniform over the workgroup
  // the query rows and scalars go out before the selection
  bf16x8_t x[4];
  if (tid < 256) attend_query_rows(x, qv, q, hg);
  const AttendQuery aq = attend_query(q, q_seq, swa_start, swa_len, T_swa);
  if (main_ch) {
    const bool writer = hg == 0 && sp == 0;
    const SelResult r = select_query<SA_NT, SEL_CAP / SA_NT>(
        q, scores, ld, n_valid, col_ids, n_cols, d, lv, kk, MODE, MODE == 0 ? idx_out : pool,
        MODE == 0 ? (int64_t)kk : (int64_t)kk * 8, pool_len, MODE == 1 ? k : 0,
        MODE == 1 ? idx_out : nullptr, vec_out, spec, writer, U.sel);
    if (tid < cps * CH_ROWS) {
      const int rr = row0 + tid;
      int32_t e = -1;
      if (rr < r.kept && rr < k) {
        const uint32_t c = r.identity ? (uint32_t)rr : r.list[rr];
        e = (MODE == 0 && col_ids) ? col_ids[(int64_t)q * ld + c] : (int32_t)c;
      }
      cid[tid] = e;
    }
    __syncthreads();
  }
  if (tid >= 256) return;                       // whole waves: the attention uses waves 0-3
  const int id0 = main_ch ? cid[tid & 63] : -1;
  const RopeArgs none = {nullptr, 0, 0.f, nullptr, {}};
  attend_body(q, hg, sp, nsplit, cps,
              [&](int r) __attribute__((always_inline)) { return cid[r - row0]; }, id0, x,
              aq, kv_codes, kv_scales, cap, k, swa_codes, swa_scale, T_swa, out, lse, part_o,
              part_ml, none, L, U.kv1);
}

// ------------------------------------------------------------ host side
static int device_cus();

// Row splits of a decode attention: as many as keep the workgroups within
// one per CU, at least one chunk each.  A workgroup holds a CU's LDS and
// registers, so workgroups past the CU count run as a second round; sizing
// the splits to one round (instead of aiming at 1024 workgroups) measured on
// MI355X: 8 queries, six attention layers at 2^19 entries, 0.220 -> 0.207 ms
// per step; 32 queries, one layer at 65,536 entries, 0.089 -> 0.079 ms.
static void attend_plan(int Q, int k, int& nsplit, int& cps) {
  const int nch = (k + CH_ROWS - 1) / CH_ROWS + AT_MAX_SWA / CH_ROWS;
  const int groups = Q * (H_ATT / AT_HG);
  int want = (device_cus() + groups - 1) / groups;
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
  hipLaunchKernelGGL(k_attend, dim3(unit_grid(Q * nsplit)), dim3(256), 0, stream, q, q_seq,
                     kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale, T_swa, swa_start,
                     swa_len, out, lse, part_o, part_ml, nsplit, cps, Q, rp);
  if (nsplit > 1)
    hipLaunchKernelGGL(k_attend_combine, dim3((unsigned)(Q * H_ATT)), dim3(128), 0, stream,
                       (const float*)part_o, (const float*)part_ml, nsplit, out, lse, rp);
  return hipGetLastError();
}

// ---- fused selection + attention
// Compute units of the current device (looked up once per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// One split per 64-row chunk: the main chunks of the top-k, then two for a
// window of up to 128 SWA rows.
static int sa_splits(int k) { return (k + CH_ROWS - 1) / CH_ROWS + AT_MAX_SWA / CH_ROWS; }
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t select_attend_ws_bytes(int Q, int64_t n_cols, int mode, int k) {
  return align256(select_ws_bytes(Q, n_cols, mode)) + attend_ws_for(Q, sa_splits(k));
}

hipError_t launch_select_attend(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                                const int32_t* col_ids, int64_t n_cols, int mode, int kk, int k,
                                int32_t* idx_out, int32_t* pool, int64_t* pool_len,
                                const uint16_t* q, const int32_t* q_seq, const uint8_t* kv_codes,
                                const uint8_t* kv_scales, int64_t cap, const uint8_t* swa_codes,
                                const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                                const int32_t* swa_len, float* out, float* lse, void* ws,
                                hipStream_t stream, bool levels_ready) {
  const LevelDesc d = select_levels(Q, n_cols, mode);
  uint32_t* lv = (uint32_t*)ws;
  const int nch = sa_splits(k);                 // one split per chunk at most
  char* part = (char*)ws + align256(select_ws_bytes(Q, n_cols, mode));
  float* part_o = (float*)part;
  // The fused kernel pays for repeating the selection in every workgroup
  // only while its workgroups fit on the device at once (one per CU): each
  // takes the fewest consecutive chunks that make them fit; past
  // SA_MAX_CPS chunks the separate kernels (same results) are faster.
  int cps = 1;
  while (cps < SA_MAX_CPS && unit_grid(Q * ((nch + cps - 1) / cps)) > (unsigned)device_cus()) ++cps;
  const int nsplit = (nch + cps - 1) / cps;
  float* part_ml = part_o + (size_t)Q * nsplit * H_ATT * D_LAT;
  if (unit_grid(Q * nsplit) > (unsigned)device_cus()) {
    hipError_t e = launch_select(scores, ld, Q, n_valid, col_ids, n_cols, kk, mode,
                                 mode == 0 ? idx_out : pool, mode == 0 ? kk : (int64_t)kk * 8,
                                 pool_len, mode == 1 ? k : 0, mode == 1 ? idx_out : nullptr, lv,
                                 stream, levels_ready);
    if (e != hipSuccess) return e;
    const RopeArgs none = {nullptr, 0, 0.f, nullptr, {}};
    return launch_attend(q, q_seq, Q, kv_codes, kv_scales, cap, idx_out, k, swa_codes, swa_scale,
                         T_swa, swa_start, swa_len, out, lse, part, attend_ws_for(Q, nch),
                         none, stream);
  }
  if (!levels_ready) {
    hipError_t e = launch_maxima(scores, ld, Q, n_valid, n_cols, d, lv, stream);
    if (e != hipSuccess) return e;
  }
  const int spec = Q <= 64;
  const int vec_out = mode == 1 && ((uintptr_t)pool & 15) == 0;
  if (mode == 0)
    hipLaunchKernelGGL(k_select_attend<0>, dim3(unit_grid(Q * nsplit)), dim3(SA_NT), 0, stream,
                       scores, ld, n_valid, col_ids, n_cols, d, (const uint32_t*)lv, kk, k, idx_out,
                       pool, pool_len, vec_out, spec, q, q_seq, kv_codes, kv_scales, cap, swa_codes,
                       swa_scale, T_swa, swa_start, swa_len, out, lse, part_o, part_ml, nsplit, cps, Q);
  else
    hipLaunchKernelGGL(k_select_attend<1>, dim3(unit_grid(Q * nsplit)), dim3(SA_NT), 0, stream,
                       scores, ld, n_valid, col_ids, n_cols, d, (const uint32_t*)lv, kk, k, idx_out,
                       pool, pool_len, vec_out, spec, q, q_seq, kv_codes, kv_scales, cap, swa_codes,
                       swa_scale, T_swa, swa_start, swa_len, out, lse, part_o, part_ml, nsplit, cps, Q);
  const RopeArgs none = {nullptr, 0, 0.f, nullptr, {}};
  hipLaunchKernelGGL(k_attend_combine, dim3((unsigned)(Q * H_ATT)), dim3(128), 0, stream,
                     (const float*)part_o, (const float*)part_ml, nsplit, out, lse, none);
  return hipGetLastError();
}

}  // namespace csa2
