// Internal launchers behind the C ABI (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Rotary position embedding around the attention, the fused RoPE -
// attention - inverse RoPE - cast kernel the report names (section 3.2):
// with dims > 0 the query's pair i = channels (512 - dims + 2i, +1) turns by
// q_pos[q] * theta^(-2i / dims) before the products and the output's by the
// opposite angle after them; out_bf16 != nullptr writes the output as bf16
// (rounded to nearest even) in place of fp32.  dims = 0 and out_bf16 =
// nullptr is the plain attention.  freq[i] = theta^(-2i / dims) in fp64,
// filled on the host.
struct RopeArgs {
  const int64_t* q_pos;
  int dims;
  float theta;
  uint16_t* out_bf16;
  double freq[32];
};

hipError_t launch_compress_quant(const uint16_t* h, const uint16_t* z, int B, int64_t T, int m,
                                 const uint16_t* w_ik, uint8_t* kv_codes, uint8_t* kv_scales,
                                 uint8_t* ik_codes, uint8_t* ik_scales, int64_t cap, int64_t e0,
                                 hipStream_t stream);

hipError_t launch_append(const uint16_t* h_new, const uint16_t* z_new, const uint16_t* swa_new,
                         int B, int m, uint16_t* tail_h, uint16_t* tail_z, int64_t* n_tok,
                         const uint16_t* w_ik, uint8_t* kv_codes, uint8_t* kv_scales,
                         uint8_t* ik_codes, uint8_t* ik_scales, int64_t cap, uint8_t* swa_codes,
                         float* swa_scale, int64_t W, int64_t* n_vis, int64_t* swa_start,
                         int32_t* swa_len, hipStream_t stream);

struct LevelDesc;
// levels != nullptr (full scans only): also writes the selection's maxima
// levels (laid out by `levels`) into lv, from the scan's epilogue when levels
// 1-2 are all there are, else by the maxima kernel after the scan.
hipError_t launch_index_score(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                              const int64_t* n_vis, const int32_t* cand, int64_t ld_cand, int Q,
                              int64_t n_cols, const uint8_t* ik_codes, const uint8_t* ik_scales,
                              int64_t cap, float* scores, int64_t ld, bool fp4q,
                              hipStream_t stream, const LevelDesc* levels = nullptr,
                              uint32_t* lv = nullptr);

// Selection: mode 0 = top-k of columns (levels down to 0), mode 1 = block
// pool (levels down to 1, blocks of 8).
size_t select_ws_bytes(int Q, int64_t n_cols, int mode);
// Bytes of the static scratch behind csa2_select_topk_noalloc, and its
// device address on the current device (looked up on the first call there).
constexpr size_t SEL_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t select_scratch(void** ptr);
// levels_ready: ws already holds the maxima levels of these scores (a scan
// with levels wrote them), so the maxima kernel is skipped.
hipError_t launch_select(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         const int32_t* col_ids, int64_t n_cols, int kk, int mode, int32_t* out,
                         int64_t out_ld, int64_t* out_len, int k2, int32_t* out2, void* ws,
                         hipStream_t stream, bool levels_ready = false);

size_t attend_ws_bytes(int Q, int k);
hipError_t launch_attend(const uint16_t* q, const int32_t* q_seq, int Q, const uint8_t* kv_codes,
                         const uint8_t* kv_scales, int64_t cap, const int32_t* idx, int k,
                         const uint8_t* swa_codes, const float* swa_scale, int64_t T_swa,
                         const int64_t* swa_start, const int32_t* swa_len, float* out, float* lse,
                         void* ws, size_t ws_bytes, const RopeArgs& rp, hipStream_t stream);

// Selection (mode 0: top-k of kk = k columns, col_ids optional; mode 1: the
// pool of kk blocks of 8 and the top-k inside it) fused with the attention
// over the top-k rows (decode batches, Q < 256); ws holds the maxima levels
// and the attention's partial states.
size_t select_attend_ws_bytes(int Q, int64_t n_cols, int mode, int k);
hipError_t launch_select_attend(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                                const int32_t* col_ids, int64_t n_cols, int mode, int kk, int k,
                                int32_t* idx_out, int32_t* pool, int64_t* pool_len,
                                const uint16_t* q, const int32_t* q_seq, const uint8_t* kv_codes,
                                const uint8_t* kv_scales, int64_t cap, const uint8_t* swa_codes,
                                const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                                const int32_t* swa_len, float* out, float* lse, void* ws,
                                hipStream_t stream, bool levels_ready = false);

hipError_t launch_attend_wide(const uint16_t* q, const int32_t* q_seq, int Q,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t cap,
                              const int32_t* idx, int k, const uint8_t* swa_codes,
                              const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                              const int32_t* swa_len, float* out, float* lse, const RopeArgs& rp,
                              hipStream_t stream);

// Counts the values of a[r][c] (r < rows, c < min(len[r], ncols)) outside
// [lo, hi) into *bad (host); synchronises the stream.
hipError_t check_range(const int32_t* a, int64_t rows, int64_t ld, const int64_t* len,
                       int64_t ncols, int64_t lo, int64_t hi, hipStream_t stream,
                       unsigned int* bad);

int selftest_count();
hipError_t launch_selftest(int32_t* counts, hipStream_t stream);

}  // namespace csa2
