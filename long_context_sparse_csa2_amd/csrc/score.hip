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
// (its half of the 128 dims) plus the 2 scale bytes of those dims, and
// converts them to bf16 with the gfx950 scaled FP4 conversion (exact for the
// power-of-two E8M0 scales).  The ReLU, the head weights and the head sum
// are applied to the accumulator in registers and the two lane halves are
// summed with one cross-lane exchange (a row-swapping permute, no LDS round
// trip), so only 4 bytes per entry are written.  Each wave keeps the bytes
// of its next two tiles in flight while it converts and multiplies the
// current one.
//
// MXFP4-query variant (report section 2.4.4: V4 trains the indexer Q and K
// for OCP MXFP4 so that the index product is an FP4 matrix multiply): the
// workgroup first quantises the query with the OCP MX rule the compressor
// applies to the indexer K (E8M0 X = 2^(floor(log2 amax) - 2) per head and
// 32-dim block, E2M1 RNE saturating) into LDS; every tile is then two gfx950
// scaled FP4 x FP4 MFMAs (32x32x64) on the raw key bytes, with no
// conversion at all.  Lane half h passes the 32 dims of block 2h + c as the
// K slice of MFMA c, for the query and the key alike (any permutation of K
// shared by both operands leaves the product unchanged), so each lane still
// streams 32 contiguous code bytes, and each lane's 32-element K slice is
// exactly one MX block with one scale byte per operand.  Products of E2M1
// values with power-of-two scales are exact; only the fp32 accumulation
// rounds.
//
// Level variant (LV): the scan also writes the first two levels of the
// selection's 8-way maxima pyramid (the maximum score key of every 8 and
// every 64 consecutive columns), so the top-k / block-pool selection that
// follows starts without a pass of its own over the scores.  A wave then
// scores its tiles in adjacent pairs (64 columns, one level-2 group); the
// 8-column maxima come from DPP lane permutations inside the tile, the
// 64-column maximum from the tile pair.
#include "common.h"
#include "launch.h"
#include "select_core.h"

namespace csa2 {

constexpr int SC_WAVES = 4;
// Two-query prefill scan (k_index_score_pair): used for launches of at
// least SC_PAIR_MIN_Q queries, 32 tiles per wave, one tile's bytes in
// flight.  Measured on MI355X against the one-query scan, at two waves per
// SIMD: 65,536-token prefill chunk scans 4.02 -> 3.81 ms per group (MXFP4
// query 2.71 -> 2.13 ms), 1,048,576-token 1.175 -> 1.038 s; at 4,096
// columns (one chunk of 4,096 queries) 76 -> 79 us with bf16 queries, which
// then kept the one-query scan, and 60 -> 54 us with MXFP4 queries; two tiles in
// flight or 16 tiles per wave ran 2-10 % slower.  Three waves per SIMD
// (tile offsets added where they are used, head weights in LDS: 145 and 116
// registers instead of 256 with spills) then took the 1,048,576-token chunk
// scans 1.04 -> 0.96 s, the 65,536-token ones 3.84 -> 3.72 ms and the
// 4,096-query MXFP4 scan 48.6 -> 45.3 us, and bf16 queries at 4,096
// columns went to pairs as well (76 -> 71 us).
constexpr int SC_PAIR_MIN_Q = 2048;
constexpr int SC_PAIR_TPW = 32, SC_PAIR_DEPTH = 1;

// Fourth word of a raw (unformatted, stride 0) buffer resource on gfx9:
// 32-bit data format, so a store is range-checked in bytes against the
// resource's record count.
constexpr int SC_RSRC_WORD3 = 0x00020000;
// Cache policy of the score stores: nontemporal.  The selection reads a
// small part of them in the next kernel, mostly from other XCDs, so they
// gain nothing from staying in this XCD's L2 (measured on MI355X: the
// 4 x 2^20 decode scan 60-64 -> 55-56 us, 58 -> 51 us after a read sweep).
// The maxima levels, which the selection reads whole and first, keep the
// default policy (nontemporal there made the decode step 1 % slower).
constexpr int SC_ST_NT = 2;

// A raw buffer resource over `bytes` bytes at p (both uniform, so the
// resource sits in scalar registers): a store at an offset past `bytes` is
// dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint64_t au = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)au, (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), SC_RSRC_WORD3);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// MXFP4 query of one workgroup: codes of head h, dims 2c and 2c+1 in byte
// c (low nibble first), and the E8M0 byte of each 32-dim block.
struct QFp4Lds {
  uint8_t codes[H_IDX][D_IDX / 2];
  uint32_t scales[H_IDX];                             // block g in byte g
};

// The workgroup's 256 threads quantise the 32 x 128 query: thread t takes
// head t / 8, block (t / 2) % 4, dims 16 (t % 2) .. +15 of that block; the
// two threads of a block share their maxima.
__device__ __forceinline__ void quant_query_fp4(const uint16_t* __restrict__ qrow, QFp4Lds& ql) {
  const int t = threadIdx.x;
  const int head = t >> 3, g = (t >> 1) & 3, sub = t & 1;
  const uint16_t* src = qrow + head * D_IDX + 32 * g + 16 * sub;
  const u32x4_t w0 = *(const u32x4_t*)src, w1 = *(const u32x4_t*)(src + 8);
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w0[i] << 16);
    v[2 * i + 1] = __uint_as_float(w0[i] & 0xFFFF0000u);
    v[8 + 2 * i] = __uint_as_float(w1[i] << 16);
    v[8 + 2 * i + 1] = __uint_as_float(w1[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  int E = -127;
  if (amax > 0.f) {
    int ex;
    (void)frexpf(amax, &ex);                          // floor(log2 amax) = ex - 1
    E = ex - 1 - 2;                                   // minus emax of E2M1
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
  }
  // E2M1(v / 2^E), round to nearest even, saturating: the gfx950 scaled
  // conversion, two values per instruction into byte sel of the word (it
  // reads only the exponent field of its scale operand, so 2^-127 is passed
  // as the subnormal with that field 0; checked against the software rule
  // on ties, saturation and the extreme scales)
  const float sc = __uint_as_float(E == -127 ? 0x00400000u : (uint32_t)(E + 127) << 23);
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[0], v[1], sc, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2], v[3], sc, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[4], v[5], sc, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[6], v[7], sc, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[8], v[9], sc, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[10], v[11], sc, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[12], v[13], sc, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[14], v[15], sc, 3);
  *(uint2*)&ql.codes[head][16 * g + 8 * sub] = make_uint2(lo, hi);
  if (sub == 0) ((uint8_t*)&ql.scales[head])[g] = (uint8_t)(E + 127);
}

// A lane offset plus a wave-uniform tile offset, as one vector add issued
// where the load or store that uses it is: left to itself the compiler
// computes the offsets of all unrolled tiles up front and keeps them in
// registers (about 80 of them at 32 tiles per wave), which limited the
// two-query scan below to two waves per SIMD.  The sum stays in the vector
// offset, which the buffer range check covers (a uniform part passed as the
// scalar offset would not be checked).
__device__ __forceinline__ int tile_off(int lane_off, int uniform_off) {
  int o;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(o) : "v"(lane_off), "s"(uniform_off));
  return o;
}

// TPW: 32-entry tiles per wave; DEPTH: tiles whose bytes are in flight ahead
// of the one being multiplied.  Workgroup chunk c starts at column
// c * chunk_stride (+ 32 per wave) and a wave's consecutive tiles are
// tile_stride columns apart; with LV (+ 64 per wave) a wave's tiles 2p and
// 2p + 1 are adjacent and its pairs tile_stride columns apart.
template <bool CAND, bool FP4Q, int TPW, int DEPTH, bool LV>
__global__ __launch_bounds__(256, 4) void k_index_score(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const int32_t* __restrict__ q_seq, const int64_t* __restrict__ n_vis,
    const int32_t* __restrict__ cand, int64_t ld_cand, int64_t nchunk, int64_t chunk_stride,
    int64_t tile_stride, int64_t n_cols,
    const uint8_t* __restrict__ ik_codes, const uint8_t* __restrict__ ik_scales, int64_t cap,
    float* __restrict__ scores, int64_t ld, LevelDesc lvd, uint32_t* __restrict__ lv) {
  static_assert(!LV || (!CAND && TPW % 2 == 0), "levels: full scans, tiles in pairs");
  // the first workgroups take the last queries: in a causal prefill chunk
  // they see the most entries, and starting the longest work first keeps it
  // out of the kernel's tail
  const int q = (int)(gridDim.x / nchunk - 1 - blockIdx.x / nchunk);
  const int64_t cbase = (int64_t)(blockIdx.x % nchunk) * chunk_stride;
  const int64_t nv0 = n_vis[q];
  // within [0, n_cols]: never past the launch's columns, and a negative
  // count scores nothing
  const int64_t nv = nv0 < 0 ? 0 : (nv0 < n_cols ? nv0 : n_cols);
  // A candidate scan has no early exit: its candidate ids, sequence and query
  // are then requested together with n_vis instead of one after the other
  // (a workgroup past n_vis scores entry 0 and its stores are dropped).
  if (!CAND && cbase >= nv) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int r = lane & 31, half = lane >> 5;
  const int64_t seq_base = (int64_t)q_seq[q] * cap;

  // A operand.  bf16: head r, dims 64*half + 8s .. +7 for step s.  MXFP4:
  // head r, blocks 2*half (MFMA 0) and 2*half + 1 (MFMA 1), scale bytes in
  // bits 0-7 and 8-15 of qsc.
  bf16x8_t a[FP4Q ? 1 : 8];
  i32x8_t qa0 = {}, qa1 = {};
  uint32_t qsc = 0;
  if constexpr (FP4Q) {
    __shared__ QFp4Lds ql;
    quant_query_fp4(q_idx + (int64_t)q * H_IDX * D_IDX, ql);
    __syncthreads();
    const u32x4_t* cp = (const u32x4_t*)&ql.codes[r][32 * half];
    const u32x4_t c0 = cp[0], c1 = cp[1];
    qa0 = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], 0, 0, 0, 0};
    qa1 = i32x8_t{(int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3], 0, 0, 0, 0};
    qsc = ql.scales[r] >> (16 * half);
  } else {
    const uint16_t* qp = q_idx + ((int64_t)q * H_IDX + r) * D_IDX + half * 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = *(const bf16x8_t*)(qp + 8 * s);
  }
  // head weight of each accumulator row this lane holds
  float wr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wr[j] = w[q * H_IDX + 8 * (j >> 2) + 4 * half + (j & 3)];

  const int32_t* crow = CAND ? cand + (int64_t)q * ld_cand : nullptr;
  float* srow = scores + (int64_t)q * ld;
  const int code_off = r * 64 + half * 32, scale_off = r * 4 + half * 2;
  // score store offset within a tile: the first lane half writes column r,
  // the second an offset past any resource (dropped)
  const int st_off = half == 0 ? r * 4 : (int)0x80000000;

  // Tile loads.  Each lane reads 32 code bytes of entry col0 + r (its lane
  // half's two MX blocks) and those blocks' two scale bytes (block 2 half in
  // bits 0-7, 2 half + 1 in bits 8-15 of scw).  A contiguous scan reads
  // through two buffer resources over the workgroup's visible entries from
  // its first column cbase on (codes and scales), so a tile's addresses are
  // one add of a wave-uniform offset per array and lanes past the row's end
  // read zeros (their scores are never stored).  The offsets fit 31 bits:
  // the host interleaves the workgroups' tiles across a row only for rows of
  // fewer than 2^24 columns (a tile requested ahead lies at most two tile
  // strides past the row), otherwise a workgroup's tiles (and the tiles it
  // requests ahead) lie within its own chunk and the next one.
  const int64_t vis_wg = nv - cbase;                  // > 0 (the workgroup has columns)
  const __amdgpu_buffer_rsrc_t rcodes = make_rsrc(
      ik_codes + (seq_base + cbase) * 64, vis_wg < ((int64_t)1 << 25) ? vis_wg * 64 : 0x7FFFFFFFll);
  const __amdgpu_buffer_rsrc_t rscales =
      make_rsrc(ik_scales + (seq_base + cbase) * 4, vis_wg * 4);
  auto load = [&](int64_t col0, u32x4_t& c0, u32x4_t& c1, uint32_t& scw) {
    if constexpr (CAND) {
      const int64_t c = col0 + r;
      const int32_t id = crow[c < n_cols ? c : n_cols - 1];   // read within the launch's columns
      const int64_t e = c < nv ? id : 0;                      // past n_vis: entry 0
      const uint8_t* cp = ik_codes + (seq_base + e) * 64 + half * 32;
      c0 = *(const u32x4_t*)cp;
      c1 = *(const u32x4_t*)(cp + 16);
      scw = *(const uint16_t*)(ik_scales + (seq_base + e) * 4 + half * 2);
    } else {
      const int d = (int)(col0 - cbase);              // < 2^25 (see above)
      const int oc = code_off + d * 64;
      c0 = __builtin_amdgcn_raw_buffer_load_b128(rcodes, oc, 0, 0);
      c1 = __builtin_amdgcn_raw_buffer_load_b128(rcodes, oc + 16, 0, 0);
      scw = __builtin_amdgcn_raw_buffer_load_b16(rscales, scale_off + d * 4, 0, 0);
    }
  };

  // The score row as a buffer resource over its nv valid columns: the
  // hardware drops a buffer store at an offset past nv * 4 bytes, so the
  // lanes without a column of their own (the second lane half, and columns
  // past the end) store without a branch, to offset 2^31 (nv * 4 < 2^31 is
  // checked on the host).
  // (readfirstlane: the resource must sit in scalar registers)
  const uint64_t sp = (uint64_t)(uintptr_t)srow;
  const uint64_t sp_u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sp) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(sp >> 32)) << 32);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)sp_u, (short)0, __builtin_amdgcn_readfirstlane((int)(nv * 4)), SC_RSRC_WORD3);

  // ring of DEPTH + 1 tiles: slot t % (DEPTH + 1) holds tile t
  u32x4_t r0[DEPTH + 1], r1[DEPTH + 1];
  uint32_t rs[DEPTH + 1];
  const int64_t step = tile_stride;
  const int64_t col_first = cbase + (int64_t)wave * (LV ? 64 : 32);
  auto col_of = [&](int t) __attribute__((always_inline)) {
    return LV ? col_first + (int64_t)(t >> 1) * step + (t & 1) * 32 : col_first + (int64_t)t * step;
  };
#pragma unroll
  for (int t = 0; t < DEPTH; ++t) {
    if (t < TPW) load(col_of(t), r0[t], r1[t], rs[t]);
  }
  // LV: the levels region as one buffer resource (its byte size fits 31
  // bits, checked on the host), the query's level-1 / level-2 rows in it
  // (uint32 units), their groups that hold a visible column, and the first
  // tile's level-1 keys and key maximum while the pair's second tile runs.
  // One store per pair writes the pair's 8 level-1 groups (lanes 8j: the
  // second tile's groups from the first lane half, the first tile's from the
  // second, both halves holding the same scores) and its level-2 group
  // (lane 1).
  const int Qn = (int)(gridDim.x / nchunk);
  const int L2 = LV && lvd.nlev >= 2;
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(
      LV ? (const void*)lv : nullptr,
      LV ? (lvd.off[1 + L2] + (int64_t)Qn * lvd.stride[1 + L2]) * 4 : 0);
  const int b1 = LV ? (int)(lvd.off[1] + (int64_t)q * lvd.stride[1]) : 0;
  const int b2 = L2 ? (int)(lvd.off[2] + (int64_t)q * lvd.stride[2]) : 0;
  const int G1 = LV ? (int)groups_at(nv, 1) : 0;
  const int G2 = L2 ? (int)groups_at(nv, 2) : 0;
  uint32_t pair_l1 = 0, pair_max = 0;
  // the level store of the pair whose first tile starts at column colA (has_b:
  // its second tile ran, its keys l1b)
  auto pair_store = [&](uint32_t l1a, uint32_t l1b, uint32_t m2, int colA, bool has_b)
      __attribute__((always_inline)) {
    const int g = (colA >> 3) + (r >> 3) + (half ? 0 : 4);
    uint32_t v = half ? l1a : l1b;
    int o = (r & 7) == 0 && g < G1 && (half || has_b) ? (b1 + g) * 4 : (int)0x80000000;
    if (lane == 1) {
      v = m2;
      o = (colA >> 6) < G2 ? (b2 + (colA >> 6)) * 4 : (int)0x80000000;
    }
    __builtin_amdgcn_raw_buffer_store_b32(v, lrs, o, 0, 0);       // cached: read first
  };
  // tile t from ring slot sl (= t mod (DEPTH + 1), a constant wherever this
  // is called); pf: first request tile t + DEPTH into its slot (a column
  // past nv re-reads the last entry, so any tile index is safe to request)
  // tail: a call from the ragged-row loop, where t is not a constant
  auto tile = [&](int t, int sl, bool pf, bool tail) __attribute__((always_inline)) {
    const int64_t col0 = col_of(t);
    if (pf) {
      const int sn = (sl + DEPTH) % (DEPTH + 1);
      load(col_of(t + DEPTH), r0[sn], r1[sn], rs[sn]);
    }
    // keep those loads ahead of this tile's work
    __builtin_amdgcn_sched_barrier(0);
    const u32x4_t c0 = r0[sl], c1 = r1[sl];
    const uint32_t scw = rs[sl];
    f32x16_t acc = {};
    if constexpr (FP4Q) {
      const i32x8_t b0 = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], 0, 0, 0, 0};
      const i32x8_t b1 = {(int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3], 0, 0, 0, 0};
      // format 4 (E2M1) for both operands; the scale operands are E8M0
      // bytes, byte 0 of qsc / scw for MFMA 0 and byte 1 for MFMA 1
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa0, b0, acc, 4, 4, 0, (int)qsc, 0,
                                                            (int)scw);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa1, b1, acc, 4, 4, 1, (int)qsc, 1,
                                                            (int)scw);
    } else {
      // 2^(c - 127) of each E8M0 byte c: c moved into the exponent field,
      // 2^-127 (a subnormal) for c = 0
      const float s_lo = __uint_as_float(max((scw << 23) & 0x7F800000u, 0x00400000u));
      const float s_hi = __uint_as_float(max((scw << 15) & 0x7F800000u, 0x00400000u));
      acc = mfma32_bf16(a[0], fp4x8_to_bf16_pow2(c0[0], s_lo), acc);
      acc = mfma32_bf16(a[1], fp4x8_to_bf16_pow2(c0[1], s_lo), acc);
      acc = mfma32_bf16(a[2], fp4x8_to_bf16_pow2(c0[2], s_lo), acc);
      acc = mfma32_bf16(a[3], fp4x8_to_bf16_pow2(c0[3], s_lo), acc);
      acc = mfma32_bf16(a[4], fp4x8_to_bf16_pow2(c1[0], s_hi), acc);
      acc = mfma32_bf16(a[5], fp4x8_to_bf16_pow2(c1[1], s_hi), acc);
      acc = mfma32_bf16(a[6], fp4x8_to_bf16_pow2(c1[2], s_hi), acc);
      acc = mfma32_bf16(a[7], fp4x8_to_bf16_pow2(c1[3], s_hi), acc);
    }
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) part += wr[j] * relu_f32(acc[j]);
    part = lanes_sum32(part);
    // (columns and their byte offsets fit 32 bits: n_cols < 2^29)
    const bool vis = r < (int)(nv - col0);
    if constexpr (CAND) {
      const int off = half == 0 && vis ? ((int)col0 + r) * 4 : (int)0x80000000;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srs, off, 0, SC_ST_NT);
    } else {                  // the second lane half at 2^31 + col0 * 4 >= nv * 4: dropped
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srs, st_off + (int)col0 * 4, 0,
                                            SC_ST_NT);
    }
    if constexpr (LV) {
      // both lane halves hold the tile's 32 scores; columns past nv count
      // as key 0, below every score's key
      uint32_t key = vis ? f32_key(part) : 0u;
      key = max(key, dpp_movu<0xb1>(key));               // quad_perm [1,0,3,2]
      key = max(key, dpp_movu<0x4e>(key));               // quad_perm [2,3,0,1]
      key = max(key, dpp_movu<0x141>(key));              // row_half_mirror: 8 columns
      const uint32_t l1 = key;
      key = max(key, dpp_movu<0x140>(key));              // row_mirror: 16 columns
      key = max(key, lanes_max16u(key));                 // the tile's 32 columns
      const bool first = (t & 1) == 0;
      if (!tail) {                                       // t is a constant here: no branch
        if (first) {
          pair_l1 = l1;
          pair_max = key;
        } else {
          pair_store(pair_l1, l1, max(pair_max, key), (int)col0 - 32, true);
        }
      } else {                                           // branch-free: a first tile stores nothing
        const int colA = (int)col0 - (first ? 0 : 32);
        pair_store(pair_l1, l1, max(pair_max, key), first ? (1 << 30) : colA, true);
        pair_l1 = first ? l1 : pair_l1;
        pair_max = first ? key : pair_max;
      }
    }
  };
  // A wave whose every tile starts before nv runs them with no branch in
  // between, so the wait before each tile covers exactly that tile's loads
  // (a branch per tile lets the compiler sink each tile's loads down to
  // their use, and makes the waits conservative).  A candidate scan always
  // does: a branch on n_vis would hold its loads back until n_vis arrives.
  // A wave that reaches nv (a causal prefill row) runs its ntv tiles in
  // branch-free groups of DEPTH + 1 (one turn of the ring, so the slots stay
  // constants), then the last ntv mod (DEPTH + 1) tiles one by one; those
  // were requested within the groups already.
  if (CAND || col_of(TPW - 1) < nv) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) tile(t, t % (DEPTH + 1), t + DEPTH < TPW, false);
  } else {
    constexpr int G = DEPTH + 1;
    const int64_t rem = nv - col_first;
    int ntv;
    if constexpr (LV) {                 // tiles before nv: first tiles p < P0, second p < P1
      const int64_t P0 = rem <= 0 ? 0 : (rem + step - 1) / step;
      const int64_t P1 = rem <= 32 ? 0 : (rem - 32 + step - 1) / step;
      ntv = (int)((P0 < TPW / 2 ? P0 : TPW / 2) + (P1 < TPW / 2 ? P1 : TPW / 2));
    } else {
      const int64_t nt64 = rem <= 0 ? 0 : (rem + step - 1) / step;
      ntv = nt64 < TPW ? (int)nt64 : TPW;
    }
    int t0 = 0;
    for (; t0 + G <= ntv; t0 += G) {
#pragma unroll
      for (int i = 0; i < G; ++i) tile(t0 + i, i, true, true);
    }
#pragma unroll
    for (int i = 0; i + 1 < G; ++i)
      if (t0 + i < ntv) tile(t0 + i, i, false, true);
    // a pair whose second tile starts past nv: its first tile's groups
    if (LV && (ntv & 1)) pair_store(pair_l1, 0u, pair_max, (int)col_of(ntv - 1), false);
  }
}

// Two queries per wave (prefill rows): the queries 2p and 2p + 1 of a causal
// prefill chunk see (nearly) the same entries, so a wave converts each
// 32-entry key tile to bf16 once and feeds it to the MFMAs of both: half the
// FP4 conversions per (query, entry), which with the epilogue bound the
// single-query scan of long rows.  With MXFP4 queries (no conversion) each
// tile's key bytes feed both queries' scaled FP4 MFMAs: half the loads per
// (query, entry) and twice the MFMA work between the waits for them.  Each query's accumulator sees
// the same operands in the same order as in the single-query scan, so the
// scores are the same bits.  Loads run to the longer of the two rows, each
// query's stores stop at its own.  A pair on two sequences (or the last,
// unpaired query) is scored one query at a time, the wave then scoring that
// query for both of its slots (the same value stored twice).
template <int TPW, int DEPTH, bool FP4Q>
__global__ __launch_bounds__(256, 3) void k_index_score_pair(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const int32_t* __restrict__ q_seq, const int64_t* __restrict__ n_vis, int Q, int64_t nchunk,
    int64_t chunk_stride, int64_t tile_stride, int64_t n_cols,
    const uint8_t* __restrict__ ik_codes, const uint8_t* __restrict__ ik_scales, int64_t cap,
    float* __restrict__ scores, int64_t ld) {
  const int p = (int)(gridDim.x / nchunk - 1 - blockIdx.x / nchunk);   // last pairs first
  const int64_t cbase = (int64_t)(blockIdx.x % nchunk) * chunk_stride;
  const int q0 = 2 * p, q1 = 2 * p + 1 < Q ? 2 * p + 1 : 2 * p;
  const bool joint = q1 != q0 && q_seq[q0] == q_seq[q1];
  const int npass = q1 != q0 && !joint ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int r = lane & 31, half = lane >> 5;
  const int code_off = r * 64 + half * 32, scale_off = r * 4 + half * 2;
  const int st_off = half == 0 ? r * 4 : (int)0x80000000;
  for (int pass = 0; pass < npass; ++pass) {
    const int qa = pass == 0 ? q0 : q1;
    const int qb = joint ? q1 : qa;
    const int64_t na0 = n_vis[qa], nb0 = n_vis[qb];
    const int64_t nva = na0 < 0 ? 0 : (na0 < n_cols ? na0 : n_cols);
    const int64_t nvb = nb0 < 0 ? 0 : (nb0 < n_cols ? nb0 : n_cols);
    const int64_t nv = nva > nvb ? nva : nvb;
    if (cbase >= nv) continue;                            // uniform
    const int64_t seq_base = (int64_t)q_seq[qa] * cap;
    bf16x8_t a0[FP4Q ? 1 : 8], a1[FP4Q ? 1 : 8];
    i32x8_t qa0[2] = {}, qa1[2] = {};           // MXFP4: the two queries' codes
    uint32_t qsc0 = 0, qsc1 = 0;
    // the two queries' head weights, read from LDS in the epilogue (in
    // registers they took 32 of the 168 a lane has at three waves per SIMD)
    __shared__ __align__(16) float wl[2][H_IDX];
    if (pass > 0) __syncthreads();                  // pass 0's weights read
    if (threadIdx.x < 2 * H_IDX)
      wl[threadIdx.x / H_IDX][threadIdx.x % H_IDX] =
          w[(threadIdx.x < H_IDX ? qa : qb) * H_IDX + threadIdx.x % H_IDX];
    {
      if constexpr (FP4Q) {
        __shared__ QFp4Lds ql[2];
        quant_query_fp4(q_idx + (int64_t)qa * H_IDX * D_IDX, ql[0]);
        quant_query_fp4(q_idx + (int64_t)qb * H_IDX * D_IDX, ql[1]);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4_t* cp = (const u32x4_t*)&ql[i].codes[r][32 * half];
          const u32x4_t c0 = cp[0], c1 = cp[1];
          i32x8_t* dst = i == 0 ? qa0 : qa1;
          dst[0] = i32x8_t{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], 0, 0, 0, 0};
          dst[1] = i32x8_t{(int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3], 0, 0, 0, 0};
        }
        qsc0 = ql[0].scales[r] >> (16 * half);
        qsc1 = ql[1].scales[r] >> (16 * half);
        __syncthreads();                    // read before a second pass rewrites them
      } else {
        const uint16_t* pa = q_idx + ((int64_t)qa * H_IDX + r) * D_IDX + half * 64;
        const uint16_t* pb = q_idx + ((int64_t)qb * H_IDX + r) * D_IDX + half * 64;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          a0[s] = *(const bf16x8_t*)(pa + 8 * s);
          a1[s] = *(const bf16x8_t*)(pb + 8 * s);
        }
      }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t sra = make_rsrc(scores + (int64_t)qa * ld, nva * 4);
    const __amdgpu_buffer_rsrc_t srb = make_rsrc(scores + (int64_t)qb * ld, nvb * 4);
    const int64_t vis_wg = nv - cbase;
    const __amdgpu_buffer_rsrc_t rcodes = make_rsrc(
        ik_codes + (seq_base + cbase) * 64, vis_wg < ((int64_t)1 << 25) ? vis_wg * 64 : 0x7FFFFFFFll);
    const __amdgpu_buffer_rsrc_t rscales = make_rsrc(ik_scales + (seq_base + cbase) * 4, vis_wg * 4);

    u32x4_t r0[DEPTH + 1], r1[DEPTH + 1];
    uint32_t rs[DEPTH + 1];
    const int64_t step = tile_stride;
    const int64_t col_first = cbase + (int64_t)wave * 32;
    auto load = [&](int t, int sl) __attribute__((always_inline)) {
      const int d = (int)(col_first + (int64_t)t * step - cbase);   // < 2^25, as in the single scan
      const int oc = tile_off(code_off, d * 64), os = tile_off(scale_off, d * 4);
      r0[sl] = __builtin_amdgcn_raw_buffer_load_b128(rcodes, oc, 0, 0);
      r1[sl] = __builtin_amdgcn_raw_buffer_load_b128(rcodes, oc + 16, 0, 0);
      rs[sl] = __builtin_amdgcn_raw_buffer_load_b16(rscales, os, 0, 0);
    };
#pragma unroll
    for (int t = 0; t < DEPTH; ++t)
      if (t < TPW) load(t, t);
    auto tile = [&](int t, int sl, bool pf) __attribute__((always_inline)) {
      if (pf) load(t + DEPTH, (sl + DEPTH) % (DEPTH + 1));
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t c0 = r0[sl], c1 = r1[sl];
      const uint32_t scw = rs[sl];
      f32x16_t acc0 = {}, acc1 = {};
      if constexpr (FP4Q) {                 // the single scan's two scaled FP4 MFMAs per query
        const i32x8_t b0 = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], 0, 0, 0, 0};
        const i32x8_t b1 = {(int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3], 0, 0, 0, 0};
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa0[0], b0, acc0, 4, 4, 0, (int)qsc0,
                                                               0, (int)scw);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa1[0], b0, acc1, 4, 4, 0, (int)qsc1,
                                                               0, (int)scw);
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa0[1], b1, acc0, 4, 4, 1, (int)qsc0,
                                                               1, (int)scw);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa1[1], b1, acc1, 4, 4, 1, (int)qsc1,
                                                               1, (int)scw);
      } else {
        const float s_lo = __uint_as_float(max((scw << 23) & 0x7F800000u, 0x00400000u));
        const float s_hi = __uint_as_float(max((scw << 15) & 0x7F800000u, 0x00400000u));
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const bf16x8_t kb = fp4x8_to_bf16_pow2(st < 4 ? c0[st] : c1[st - 4], st < 4 ? s_lo : s_hi);
          acc0 = mfma32_bf16(a0[st], kb, acc0);
          acc1 = mfma32_bf16(a1[st], kb, acc1);
        }
      }
      float pa = 0.f, pb = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4_t wa = *(const f32x4_t*)&wl[0][8 * m + 4 * half];
        const f32x4_t wb = *(const f32x4_t*)&wl[1][8 * m + 4 * half];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pa += wa[i] * relu_f32(acc0[4 * m + i]);
          pb += wb[i] * relu_f32(acc1[4 * m + i]);
        }
      }
      pa = lanes_sum32(pa);
      pb = lanes_sum32(pb);
      const int so = tile_off(st_off, (int)(col_first + (int64_t)t * step) * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pa), sra, so, 0, SC_ST_NT);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pb), srb, so, 0, SC_ST_NT);
    };
    // the single-query scan's loop shape: all tiles branch-free when the
    // wave's last tile starts before nv, else ring-turn groups of DEPTH + 1
    if (col_first + (int64_t)(TPW - 1) * step < nv) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) tile(t, t % (DEPTH + 1), t + DEPTH < TPW);
    } else {
      constexpr int G = DEPTH + 1;
      const int64_t rem = nv - col_first;
      const int64_t nt64 = rem <= 0 ? 0 : (rem + step - 1) / step;
      const int ntv = nt64 < TPW ? (int)nt64 : TPW;
      int t0 = 0;
      for (; t0 + G <= ntv; t0 += G) {
#pragma unroll
        for (int i = 0; i < G; ++i) tile(t0 + i, i, true);
      }
#pragma unroll
      for (int i = 0; i + 1 < G; ++i)
        if (t0 + i < ntv) tile(t0 + i, i, false);
    }
  }
}

template <bool CAND, int TPW, int DEPTH, bool LV>
static void launch_variant(bool fp4q, dim3 grid, hipStream_t stream, const uint16_t* q_idx,
                           const float* w,
                           const int32_t* q_seq, const int64_t* n_vis, const int32_t* cand,
                           int64_t ld_cand, int64_t nchunk, int64_t chunk_stride,
                           int64_t tile_stride, int64_t n_cols,
                           const uint8_t* ik_codes, const uint8_t* ik_scales, int64_t cap,
                           float* scores, int64_t ld, const LevelDesc& lvd, uint32_t* lv) {
  if (fp4q)
    hipLaunchKernelGGL((k_index_score<CAND, true, TPW, DEPTH, LV>), grid, dim3(256), 0, stream,
                       q_idx, w, q_seq, n_vis, cand, ld_cand, nchunk, chunk_stride, tile_stride,
                       n_cols, ik_codes, ik_scales, cap, scores, ld, lvd, lv);
  else
    hipLaunchKernelGGL((k_index_score<CAND, false, TPW, DEPTH, LV>), grid, dim3(256), 0, stream,
                       q_idx, w, q_seq, n_vis, cand, ld_cand, nchunk, chunk_stride, tile_stride,
                       n_cols, ik_codes, ik_scales, cap, scores, ld, lvd, lv);
}

hipError_t launch_index_score(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                              const int64_t* n_vis, const int32_t* cand, int64_t ld_cand, int Q,
                              int64_t n_cols, const uint8_t* ik_codes, const uint8_t* ik_scales,
                              int64_t cap, float* scores, int64_t ld, bool fp4q,
                              hipStream_t stream, const LevelDesc* levels, uint32_t* lv) {
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
  // The scan writes the selection's levels 1 and 2 itself when they are all
  // the selection needs and its waves take tiles in pairs; otherwise the
  // maxima kernel derives them from the scores afterwards.
  const LevelDesc none = {};
  const bool lv_scan = levels && !cand && tpw >= 2 && levels->nlev >= 1 && levels->nlev <= 2 &&
                       (levels->off[levels->nlev] + (int64_t)Q * levels->stride[levels->nlev]) * 4 <
                           ((int64_t)1 << 31);
  const LevelDesc& lvd = levels ? *levels : none;
  // Long scans (>= 128 chunks per query) interleave the workgroups' tiles:
  // workgroup g takes 128-column slices g, g + nchunk, g + 2 nchunk, ...
  // (256-column slices of tile pairs with levels), so at any moment the
  // workgroups of a query read one contiguous window instead of nchunk
  // windows a fixed power-of-two stride apart (measured on MI355X: 2-7 %
  // faster at 512K-1M entries, 3-5 % slower at 64K).
  const bool inter = nchunk >= 128 && n_cols < ((int64_t)1 << 24);
  const int64_t slice = (int64_t)SC_WAVES * 32 * (lv_scan ? 2 : 1);
  const int64_t cs = inter ? slice : cols;
  const int64_t ts = inter ? nchunk * slice : slice;
#define CSA2_SCORE_CASE(T, D)                                                          \
  case T:                                                                             \
    if (cand)                                                                         \
      launch_variant<true, T, D, false>(fp4q, grid, stream, q_idx, w, q_seq, n_vis, cand, \
                                        ld_cand, nchunk, cs, ts, n_cols, ik_codes,    \
                                        ik_scales, cap, scores, ld, lvd, lv);         \
    else if (lv_scan)                                                                 \
      launch_variant<false, T, D, (T % 2 == 0)>(fp4q, grid, stream, q_idx, w, q_seq,  \
                                                n_vis, cand, ld_cand, nchunk, cs, ts, \
                                                n_cols, ik_codes, ik_scales, cap,     \
                                                scores, ld, lvd, lv);                 \
    else                                                                              \
      launch_variant<false, T, D, false>(fp4q, grid, stream, q_idx, w, q_seq, n_vis,  \
                                         cand, ld_cand, nchunk, cs, ts, n_cols,       \
                                         ik_codes, ik_scales, cap, scores, ld, lvd, lv); \
    break;
  // Prefill chunks: two queries per wave share each key tile's conversion
  // (bf16 query) or its loads (MXFP4 query); same scores, bit for bit
  const int64_t P = ((int64_t)Q + 1) / 2;
  constexpr int64_t pcols = (int64_t)SC_WAVES * SC_PAIR_TPW * 32;
  const int64_t pchunk = (n_cols + pcols - 1) / pcols;
  const bool pairs = !cand && !lv_scan && Q >= SC_PAIR_MIN_Q &&
                     n_cols > 0 && P * pchunk >= 1024;
  if (pairs) {
    const bool pinter = pchunk >= 128 && n_cols < ((int64_t)1 << 24);
    const int64_t pslice = (int64_t)SC_WAVES * 32;
    if (fp4q)
      hipLaunchKernelGGL((k_index_score_pair<SC_PAIR_TPW, SC_PAIR_DEPTH, true>),
                         dim3((unsigned)(pchunk * P)), dim3(256), 0, stream, q_idx, w, q_seq,
                         n_vis, Q, pchunk, pinter ? pslice : pcols,
                         pinter ? pchunk * pslice : pslice, n_cols, ik_codes, ik_scales, cap,
                         scores, ld);
    else
      hipLaunchKernelGGL((k_index_score_pair<SC_PAIR_TPW, SC_PAIR_DEPTH, false>),
                         dim3((unsigned)(pchunk * P)), dim3(256), 0, stream, q_idx, w, q_seq,
                         n_vis, Q, pchunk, pinter ? pslice : pcols,
                         pinter ? pchunk * pslice : pslice, n_cols, ik_codes, ik_scales, cap,
                         scores, ld);
    tpw = 0;                                                    // launched
  }
  switch (tpw) {
    case 0:
      break;
    CSA2_SCORE_CASE(32, 2)
    CSA2_SCORE_CASE(16, 2)
    CSA2_SCORE_CASE(8, 2)
    CSA2_SCORE_CASE(2, 1)
    default:
    CSA2_SCORE_CASE(1, 1)
  }
#undef CSA2_SCORE_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (levels && !lv_scan && levels->nlev > 0)
    e = launch_maxima(scores, ld, Q, n_vis, n_cols, *levels, lv, stream);
  return e;
}

}  // namespace csa2
