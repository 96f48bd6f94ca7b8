// Steps a8 + a9 for many queries at once (prefill): one 256-thread
// workgroup per query covering all 64 heads, so every gathered row is read
// and dequantised once for the whole query.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3: each query attends to
// its selected main-KV entries plus the layer's SWA rows, the 512-d latent
// being both key and value; section 2.4.4: FP4 main KV dequantised before
// attention, FP8 SWA KV.
//
// The workgroup holds about 80 KB of LDS, so two queries' workgroups share
// a CU and their phases interleave: one's softmax and staging run while the
// other's MFMAs and LDS reads do.  Per 64-row chunk (main-KV chunks first,
// then SWA chunks, so each chunk has one row type):
//   staging  thread t loads the raw bytes of row t & 63, dims 128 (t >> 6)
//            .. +127 (its row id one chunk ahead) and writes them
//            dequantised to fp16 in LDS (attend_stage.h);
//            SWA rows are staged unscaled, once: their row scale multiplies
//            the scores and P
//   S^T      64 rows x 16 heads per wave (wave w: heads 16w .. +15), fp16
//            MFMA 16x16x32 with the staged rows as A and the query, in
//            registers as fp16 (each head scaled by a power of two, undone
//            on S), as B; a lane then holds one head's scores for 16 rows
//   softmax  per head within the wave (in-lane, then the lanes xor 16 and
//            32 by row-swapping permutes); the reference max only moves
//            when a chunk beats it by more than e^8, so O is rescaled in
//            few chunks; P^T and the per-head rescale factors go to LDS
//   O^T += V^T P^T  512 dims x 64 heads, wave w: dims 128w .. +127 for all
//            heads, so every staged value is read once; V^T through
//            transposing LDS reads of the staged rows, P^T from LDS
#include "common.h"
#include "launch.h"
#include "attend_stage.h"

namespace csa2 {

constexpr int AW_THREADS = 256;
constexpr int AW_PAD = 8;              // fp16 padding of a P^T row
constexpr int AW_MAX_SWA = 128;        // largest SWA window per query
constexpr float AW_LAZY = 8.f;         // slack of the softmax reference max (natural log)

// ROPE: the query is turned before QK^T and the output turned back (the
// variant without it leaves the low query terms out of the registers).
template <bool ROPE>
__global__ __launch_bounds__(AW_THREADS, 2) void k_attend_wide(
    const uint16_t* __restrict__ qv, const int32_t* __restrict__ q_seq,
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t cap,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa_codes,
    const float* __restrict__ swa_scale, int64_t T_swa, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float* __restrict__ out, float* __restrict__ lse,
    RopeArgs rp) {
  __shared__ __align__(16) _Float16 kv[CH_ROWS * KV_LD];           // the chunk's rows (K = V)
  __shared__ __align__(16) _Float16 pt[H_ATT][CH_ROWS + AW_PAD];   // P^T (SWA rows: times the row scale)
  __shared__ __align__(16) float rowsc[CH_ROWS];                   // score scale of a row; -1 = no row
  __shared__ float head_a[H_ATT];                                  // this chunk's O rescale per head
  __shared__ float head_l[H_ATT];                                  // softmax sums at the end
  __shared__ int moved_w[4];                                       // a wave's heads moved their max
  __shared__ f32x2_t rcs[ROPE_MAX_PAIRS];                          // RoPE (cos, sin) per pair

  const int q = gridDim.x - 1 - blockIdx.x;        // last queries (most rows when causal) first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: scalar registers
  const int r16 = lane & 15, qd = lane >> 4;
  const int head = 16 * wave + r16;                      // S^T and softmax: this lane's head
  const int64_t seq = q_seq[q];
  const int64_t sst = swa_start[q];
  int64_t sl64 = swa_len[q];
  if (sst < 0 || sst >= T_swa) sl64 = 0;                     // ring: start must be a slot
  else if (sl64 > T_swa) sl64 = T_swa;                       // at most one lap
  const int sl = sl64 < 0 ? 0 : (sl64 > AW_MAX_SWA ? AW_MAX_SWA : (int)sl64);
  const int nmc = (k + CH_ROWS - 1) / CH_ROWS;
  const int nch = nmc + (sl + CH_ROWS - 1) / CH_ROWS;
  const int srow = tid & 63, spart = wave;              // this thread's staging share

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

  // ---- row ids one chunk ahead (the raw bytes are loaded at staging: the
  // other workgroup on the CU computes meanwhile)
  int cur_e = entry_of(0);

  // ---- query of head `head` as the B operand: dims 32 s + 8 qd .. +7 for step s
  f16x8_t a[16];
  f16x8_t alo[2];                 // with RoPE: low terms of steps 14 and 15
  float hinv;
  {
    const uint16_t* qp = qv + ((int64_t)q * H_ATT + head) * D_LAT + 8 * qd;
    bf16x8_t x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = *(const bf16x8_t*)(qp + 32 * s);
    if (ROPE) rope_table<AW_THREADS>(rp, q, rcs);  // while the query bytes are in flight
    float xf[16][8];
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) xf[s][j] = (float)x[s][j];
    if (ROPE && rp.dims > 0) {
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
    mx = lanes_max32(lanes_max16(mx));
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
    hinv = ldexpf(1.f, -e);
  }
  // O^T tiles: dims 128 wave + 16 t + 4 qd + j, head 16 g + r16
  f32x4_t o[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) o[t][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;                 // of head `head` (equal in its 4 lanes)

  for (int ch = 0; ch < nch; ++ch) {
    const bool is_main = ch < nmc;
    // ---- this chunk's rows, dequantised, into LDS
    {
      const int64_t off = row_of(ch, cur_e);
      cur_e = entry_of(ch + 1);
      const bool valid = off >= 0;
      RawShare<AW_THREADS> raw;
      load_share<AW_THREADS>(raw, is_main, valid ? off : (is_main ? seq * cap : seq * T_swa + sst),
                             spart, kv_codes, kv_scales, swa_codes);
      const float sg = (!is_main && valid) ? swa_scale[off] : 1.f;
      if (tid < CH_ROWS) rowsc[tid] = valid ? sg : -1.f;
      store_share<AW_THREADS, false>(raw, is_main, valid, sg, kv, nullptr, srow, spart);
    }
    __syncthreads();

    // ---- S^T for rows 16 rt + 4 qd + j, head `head`
    float s[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 16; ++st) acc = mfma16_f16(qk_b(kv, 16 * rt + r16, st, qd), a[st], acc);
      if (ROPE && rp.dims > 0) {
#pragma unroll
        for (int st = 0; st < 2; ++st) acc = mfma16_f16(qk_b(kv, 16 * rt + r16, 14 + st, qd), alo[st], acc);
      }
      const f32x4_t rs = *(const f32x4_t*)&rowsc[16 * rt + 4 * qd];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[rt][j] = rs[j] >= 0.f ? acc[j] * hinv * rs[j] : -INFINITY;
    }

    // ---- online softmax of head `head` over the chunk's 64 rows
    float cm = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) cm = fmaxf(cm, s[rt][j]);
    cm = lanes_max32(lanes_max16(cm));
    // the reference max moves only when a chunk exceeds it by more than
    // AW_LAZY (P then stays below e^AW_LAZY, far inside fp16)
    const float m_new = cm > m_run + AW_LAZY ? cm : m_run;
    const bool moved = m_new != m_run;
    float alpha = 1.f, psum = 0.f;
    const f32x4_t* rsv = (const f32x4_t*)rowsc;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const f32x4_t rs = rsv[4 * rt + qd];
      f16x4_t pv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = m_new == -INFINITY ? 0.f : exp_hw(s[rt][j] - m_new);   // masked rows: 0
        psum += p;
        pv[j] = (_Float16)(is_main ? p : p * fmaxf(rs[j], 0.f));     // SWA: V is unscaled
      }
      *(f16x4_t*)&pt[head][16 * rt + 4 * qd] = pv;
    }
    if (m_new != -INFINITY) alpha = exp_hw(m_run - m_new);          // 0 when m_run is -inf
    psum = lanes_sum32(lanes_sum16(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (qd == 0) head_a[head] = alpha;
    const uint64_t mv = __ballot(moved);
    if (lane == 0) moved_w[wave] = mv != 0;
    __syncthreads();

    // ---- O^T += V^T P^T: dims 128 wave .. +127, all 64 heads
    if (moved_w[0] | moved_w[1] | moved_w[2] | moved_w[3]) {     // uniform
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float al = head_a[16 * g + r16];
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t][g] *= al;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {                 // rows 32 kk .. +31
      f16x8_t pb[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) pb[g] = *(const f16x8_t*)&pt[16 * g + r16][32 * kk + 8 * qd];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f16x8_t va = pv_b(kv, 32 * kk, 128 * wave + 16 * t, lane);
#pragma unroll
        for (int g = 0; g < 4; ++g) o[t][g] = mfma16_f16(va, pb[g], o[t][g]);
      }
    }
    __syncthreads();
  }

  // ---- normalise by each head's sum and write (RoPE channels turned back)
  if (qd == 0) head_l[head] = l_run;
  if (lse && qd == 0)
    lse[(int64_t)q * H_ATT + head] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int hh = 16 * g + r16;
    const float L = head_l[hh];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t row = ((int64_t)q * H_ATT + hh) * D_LAT;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int d0 = 128 * wave + 16 * t + 4 * qd;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = o[t][g][j] * inv;
      if (ROPE && rp.dims > 0 && 128 * wave + 16 * t + 15 >= D_LAT - rp.dims) {   // uniform per wave
        rope_pair(v[0], v[1], d0, rp.dims, rcs, -1.f);
        rope_pair(v[2], v[3], d0 + 2, rp.dims, rcs, -1.f);
      }
      if (rp.out_bf16) {
        const uint32_t lo = (uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16);
        const uint32_t hi = (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16);
        *(uint2*)(rp.out_bf16 + row + d0) = make_uint2(lo, hi);
      } else {
        *(f32x4_t*)(out + row + d0) = f32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

hipError_t launch_attend_wide(const uint16_t* q, const int32_t* q_seq, int Q,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
                              const int32_t* idx, int k, const uint8_t* swa_codes,
                              const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                              const int32_t* swa_len, float* out, float* lse, const RopeArgs& rp,
                              hipStream_t stream) {
  if (rp.dims > 0)
    hipLaunchKernelGGL(k_attend_wide<true>, dim3((unsigned)Q), dim3(AW_THREADS), 0, stream, q,
                       q_seq, kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale, T_swa,
                       swa_start, swa_len, out, lse, rp);
  else
    hipLaunchKernelGGL(k_attend_wide<false>, dim3((unsigned)Q), dim3(AW_THREADS), 0, stream, q,
                       q_seq, kv_codes, kv_scales, cap, idx, k, swa_codes, swa_scale, T_swa,
                       swa_start, swa_len, out, lse, rp);
  return hipGetLastError();
}

}  // namespace csa2
