// C ABI of libcsa2: host-side validation and dispatch to the kernels.
// Every check runs before anything is launched; see include/csa2.h for the
// contract of each entry point.
#include "csa2.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "launch.h"
#include "select_core.h"

static_assert(CSA2_NOALLOC_SCRATCH_BYTES == csa2::SEL_SCRATCH_BYTES,
              "the header states the static scratch size");

namespace {

thread_local char g_err[512];

csa2_status fail(csa2_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
// an optional array (NULL allowed) aligned to `a` bytes when given
bool al0(const void* p, uintptr_t a) { return !p || al(p, a); }

csa2_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA2_OK;
  return fail(CSA2_EHIP, "%s: %s", what, hipGetErrorString(e));
}

csa2_status check_cache(const csa2_cache* c) {
  if (!c) return fail(CSA2_EINVAL, "cache is NULL");
  if (!c->kv_codes || !c->kv_scales || !c->ik_codes || !c->ik_scales)
    return fail(CSA2_EINVAL, "cache has a NULL array");
  if (!al(c->kv_codes, 16) || !al(c->kv_scales, 16) || !al(c->ik_codes, 16) ||
      !al(c->ik_scales, 16))
    return fail(CSA2_EINVAL, "cache arrays must be 16-byte aligned");
  if (c->cap <= 0) return fail(CSA2_EINVAL, "cache cap=%lld must be > 0", (long long)c->cap);
  if (c->batch < 0) return fail(CSA2_EINVAL, "cache batch=%lld must be >= 0", (long long)c->batch);
  return CSA2_OK;
}

// CSA2_CHECK=1 in the environment: device index arrays are range-checked
// (synchronously) before the kernels that use them run.
bool device_checks() {
  const char* v = getenv("CSA2_CHECK");
  return v && strcmp(v, "1") == 0;
}

csa2_status check_indices(const char* what, const int32_t* a, int64_t rows, int64_t ld,
                          const int64_t* len, int64_t ncols, int64_t lo, int64_t hi,
                          void* stream) {
  unsigned int bad = 0;
  const hipError_t e = csa2::check_range(a, rows, ld, len, ncols, lo, hi, (hipStream_t)stream, &bad);
  if (e != hipSuccess) return fail(CSA2_EHIP, "CSA2_CHECK %s: %s", what, hipGetErrorString(e));
  if (bad)
    return fail(CSA2_EINVAL, "CSA2_CHECK: %u value(s) of %s outside [%lld, %lld)", bad, what,
                (long long)lo, (long long)hi);
  return CSA2_OK;
}

#define CHECKED(call)                        \
  do {                                       \
    const csa2_status st_ = (call);          \
    if (st_ != CSA2_OK) return st_;          \
  } while (0)

#define REQ(cond, ...)                                   \
  do {                                                   \
    if (!(cond)) return fail(CSA2_EINVAL, __VA_ARGS__);  \
  } while (0)

}  // namespace

extern "C" {

const char* csa2_status_string(int s) {
  switch (s) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_EINVAL: return "CSA2_EINVAL";
    case CSA2_EUNSUPPORTED: return "CSA2_EUNSUPPORTED";
    case CSA2_EWORKSPACE: return "CSA2_EWORKSPACE";
    case CSA2_EHIP: return "CSA2_EHIP";
    default: return "CSA2_UNKNOWN";
  }
}

const char* csa2_last_error(void) { return g_err; }

csa2_status csa2_compress_quant(const uint16_t* h, const uint16_t* z, int B, int64_t T, int m,
                                const uint16_t* w_ik, const csa2_cache* dst, int64_t e0,
                                void* stream) {
  g_err[0] = 0;
  REQ(h && w_ik, "h and w_ik must not be NULL");
  const csa2_status cs = check_cache(dst);
  if (cs != CSA2_OK) return cs;
  REQ(B > 0 && B <= 65535, "B=%d must be in [1, 65535]", B);
  REQ(T > 0, "T=%lld must be > 0", (long long)T);
  REQ(m >= 1 && m <= 16, "m=%d must be in [1, 16]", m);
  REQ(T % m == 0, "T=%lld is not a multiple of m=%d", (long long)T, m);
  REQ(m == 1 || z, "z must be given when m > 1");
  REQ(e0 >= 0 && e0 + T / m <= dst->cap, "entries [%lld, %lld) exceed cap=%lld", (long long)e0,
      (long long)(e0 + T / m), (long long)dst->cap);
  REQ(al(h, 16) && (!z || al(z, 16)) && al(w_ik, 16), "h, z, w_ik must be 16-byte aligned");
  return hip_status(csa2::launch_compress_quant(h, m == 1 ? nullptr : z, B, T, m, w_ik,
                                                dst->kv_codes, dst->kv_scales, dst->ik_codes,
                                                dst->ik_scales, dst->cap, e0,
                                                (hipStream_t)stream),
                    "csa2_compress_quant launch");
}

csa2_status csa2_decode_append(const uint16_t* h_new, const uint16_t* z_new,
                               const uint16_t* swa_new, int B, const uint16_t* w_ik,
                               const csa2_cache* cache, const csa2_state* state, int64_t* n_vis,
                               int64_t* swa_start, int32_t* swa_len, void* stream) {
  g_err[0] = 0;
  REQ(h_new && w_ik && state, "h_new, w_ik, state must not be NULL");
  const csa2_status cs = check_cache(cache);
  if (cs != CSA2_OK) return cs;
  const int m = state->m;
  const int64_t W = state->W;
  REQ(B > 0 && B <= 65535, "B=%d must be in [1, 65535]", B);
  REQ(m >= 1 && m <= 16, "state->m=%d must be in [1, 16]", m);
  REQ(W >= 0 && W <= CSA2_MAX_SWA, "state->W=%lld must be in [0, %d]", (long long)W,
      CSA2_MAX_SWA);
  REQ(state->n_tok, "state->n_tok must not be NULL");
  REQ(m == 1 || (z_new && state->tail_h && state->tail_z),
      "z_new, state->tail_h and state->tail_z must be given when m > 1");
  REQ(W == 0 || (swa_new && state->swa_codes && state->swa_scale),
      "swa_new, state->swa_codes and state->swa_scale must be given when W > 0");
  REQ(al(h_new, 16) && (!z_new || al(z_new, 16)) && (!swa_new || al(swa_new, 16)) &&
          al(w_ik, 16) && (!state->tail_h || al(state->tail_h, 16)) &&
          (!state->tail_z || al(state->tail_z, 16)) && al(state->n_tok, 8) &&
          (!state->swa_codes || al(state->swa_codes, 16)) &&
          (!state->swa_scale || al(state->swa_scale, 4)),
      "h_new, z_new, swa_new, w_ik and the state arrays must be 16-byte aligned");
  REQ(al0(n_vis, 8) && al0(swa_start, 8) && al0(swa_len, 4),
      "n_vis and swa_start must be 8-byte aligned, swa_len 4-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const uint16_t* zn = m == 1 ? nullptr : z_new;
  return hip_status(csa2::launch_append(h_new, zn, W > 0 ? swa_new : nullptr, B, m,
                                        state->tail_h, state->tail_z, state->n_tok, w_ik,
                                        cache->kv_codes, cache->kv_scales, cache->ik_codes,
                                        cache->ik_scales, cache->cap, state->swa_codes,
                                        state->swa_scale, W, n_vis, swa_start, swa_len, st),
                    "csa2_decode_append launch");
}

static csa2_status index_score_common(const uint16_t* q_idx, const float* w,
                                      const int32_t* q_seq, const int64_t* n_vis,
                                      const int32_t* cand, int64_t ld_cand, int Q, int64_t n_cols,
                                      const csa2_cache* src, float* scores, int64_t ld,
                                      void* stream, bool fp4q,
                                      const csa2::LevelDesc* levels = nullptr,
                                      uint32_t* lv = nullptr) {
  REQ(q_idx && w && q_seq && n_vis && scores, "q_idx, w, q_seq, n_vis, scores must not be NULL");
  const csa2_status cs = check_cache(src);
  if (cs != CSA2_OK) return cs;
  REQ(Q > 0, "Q=%d must be > 0", Q);
  REQ(n_cols >= 0 && n_cols < ((int64_t)1 << 29), "n_cols=%lld must be in [0, 2^29)",
      (long long)n_cols);
  REQ(ld >= n_cols, "ld=%lld < n_cols=%lld", (long long)ld, (long long)n_cols);
  REQ(!cand || ld_cand >= n_cols, "ld_cand=%lld < n_cols=%lld", (long long)ld_cand,
      (long long)n_cols);
  REQ(cand || n_cols <= src->cap, "n_cols=%lld exceeds cap=%lld", (long long)n_cols,
      (long long)src->cap);
  REQ(al(q_idx, 16) && al(w, 4) && al(q_seq, 4) && al(n_vis, 8) && al0(cand, 4) &&
          al(scores, 4),
      "q_idx must be 16-byte aligned, n_vis 8-byte aligned, w, q_seq, cand and scores "
      "4-byte aligned");
  if (n_cols == 0) return CSA2_OK;
  REQ((n_cols + 1023) / 1024 * (int64_t)Q < (int64_t)1 << 31, "launch too large");
  if (device_checks()) {
    CHECKED(check_indices("q_seq", q_seq, 1, Q, nullptr, Q, 0,
                          src->batch > 0 ? src->batch : (int64_t)INT32_MAX, stream));
    if (cand)
      CHECKED(check_indices("cand", cand, Q, ld_cand, n_vis, n_cols, 0, src->cap, stream));
  }
  return hip_status(csa2::launch_index_score(q_idx, w, q_seq, n_vis, cand, ld_cand, Q, n_cols,
                                             src->ik_codes, src->ik_scales, src->cap, scores, ld,
                                             fp4q, (hipStream_t)stream, levels, lv),
                    levels ? "csa2_index_score_levels launch"
                           : fp4q ? "csa2_index_score_fp4q launch" : "csa2_index_score launch");
}

csa2_status csa2_index_score(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                             const int64_t* n_vis, const int32_t* cand, int64_t ld_cand, int Q,
                             int64_t n_cols, const csa2_cache* src, float* scores, int64_t ld,
                             void* stream) {
  g_err[0] = 0;
  return index_score_common(q_idx, w, q_seq, n_vis, cand, ld_cand, Q, n_cols, src, scores, ld,
                            stream, false);
}

csa2_status csa2_index_score_fp4q(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                  const int64_t* n_vis, const int32_t* cand, int64_t ld_cand,
                                  int Q, int64_t n_cols, const csa2_cache* src, float* scores,
                                  int64_t ld, void* stream) {
  g_err[0] = 0;
  return index_score_common(q_idx, w, q_seq, n_vis, cand, ld_cand, Q, n_cols, src, scores, ld,
                            stream, true);
}

csa2_status csa2_index_score_levels(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                    const int64_t* n_vis, int Q, int64_t n_cols,
                                    const csa2_cache* src, float* scores, int64_t ld, int fp4q,
                                    int n_blocks, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  REQ(Q > 0, "Q=%d must be > 0", Q);
  REQ(n_blocks >= 0 && n_blocks <= CSA2_MAX_K, "n_blocks=%d must be in [0, %d]", n_blocks,
      CSA2_MAX_K);
  REQ(n_cols >= 0 && n_cols <= CSA2_MAX_COLS, "n_cols=%lld must be in [0, %d]",
      (long long)n_cols, CSA2_MAX_COLS);
  const int mode = n_blocks > 0 ? 1 : 0;
  // (no levels at all when the selection takes the scores directly)
  const size_t need = csa2::select_ws_bytes(Q, n_cols, mode);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA2_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0,
                need);
  REQ(!ws || al(ws, 256), "ws must be 256-byte aligned");
  const csa2::LevelDesc d = csa2::select_levels(Q, n_cols, mode);
  return index_score_common(q_idx, w, q_seq, n_vis, nullptr, 0, Q, n_cols, src, scores, ld,
                            stream, fp4q != 0, &d, (uint32_t*)ws);
}

static csa2_status select_common(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                                 const int32_t* col_ids, int64_t n_cols, int kk, void* ws,
                                 size_t ws_bytes, int mode) {
  REQ(scores && n_valid, "scores and n_valid must not be NULL");
  REQ(Q > 0, "Q=%d must be > 0", Q);
  REQ(kk >= 1 && kk <= CSA2_MAX_K, "k=%d must be in [1, %d]", kk, CSA2_MAX_K);
  REQ(n_cols >= 0 && n_cols <= CSA2_MAX_COLS, "n_cols=%lld must be in [0, %d]",
      (long long)n_cols, CSA2_MAX_COLS);
  REQ(ld >= n_cols && ld > 0, "ld=%lld < n_cols=%lld", (long long)ld, (long long)n_cols);
  REQ(al(scores, 4) && al(n_valid, 8) && al0(col_ids, 4),
      "scores and col_ids must be 4-byte aligned, n_valid 8-byte aligned");
  const size_t need = csa2::select_ws_bytes(Q, n_cols, mode);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA2_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0,
                need);
  REQ(!ws || al(ws, 16), "ws must be 16-byte aligned");
  return CSA2_OK;
}

csa2_status csa2_select_topk(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                             const int32_t* col_ids, int64_t n_cols, int k, int32_t* out,
                             void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  REQ(out && al(out, 4), "out must not be NULL and 4-byte aligned");
  const csa2_status st =
      select_common(scores, ld, Q, n_valid, col_ids, n_cols, k, ws, ws_bytes, 0);
  if (st != CSA2_OK) return st;
  return hip_status(csa2::launch_select(scores, ld, Q, n_valid, col_ids, n_cols, k, 0, out, k,
                                        nullptr, 0, nullptr, ws, (hipStream_t)stream),
                    "csa2_select_topk launch");
}

csa2_status csa2_select_topk_levels(const float* scores, int64_t ld, int Q,
                                    const int64_t* n_valid, const int32_t* col_ids,
                                    int64_t n_cols, int k, int32_t* out, void* ws,
                                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  REQ(out && al(out, 4), "out must not be NULL and 4-byte aligned");
  REQ(!col_ids, "col_ids must be NULL (the levels are those of a full scan)");
  const csa2_status st =
      select_common(scores, ld, Q, n_valid, col_ids, n_cols, k, ws, ws_bytes, 0);
  if (st != CSA2_OK) return st;
  return hip_status(csa2::launch_select(scores, ld, Q, n_valid, col_ids, n_cols, k, 0, out, k,
                                        nullptr, 0, nullptr, ws, (hipStream_t)stream, true),
                    "csa2_select_topk_levels launch");
}

csa2_status csa2_select_topk_noalloc(const float* scores, int64_t ld, int Q,
                                     const int64_t* n_valid, const int32_t* col_ids,
                                     int64_t n_cols, int k, int32_t* out, void* stream) {
  g_err[0] = 0;
  REQ(out && al(out, 4), "out must not be NULL and 4-byte aligned");
  REQ(scores && n_valid, "scores and n_valid must not be NULL");
  REQ(Q > 0, "Q=%d must be > 0", Q);
  REQ(k >= 1 && k <= CSA2_MAX_K, "k=%d must be in [1, %d]", k, CSA2_MAX_K);
  REQ(n_cols >= 0 && n_cols <= CSA2_MAX_COLS, "n_cols=%lld must be in [0, %d]",
      (long long)n_cols, CSA2_MAX_COLS);
  REQ(ld >= n_cols && ld > 0, "ld=%lld < n_cols=%lld", (long long)ld, (long long)n_cols);
  REQ(al(scores, 4) && al(n_valid, 8) && al0(col_ids, 4),
      "scores and col_ids must be 4-byte aligned, n_valid 8-byte aligned");
  const size_t need = csa2::select_ws_bytes(Q, n_cols, 0);
  if (need > csa2::SEL_SCRATCH_BYTES)
    return fail(CSA2_EUNSUPPORTED,
                "Q=%d x n_cols=%lld needs %zu bytes of scratch, more than the %zu-byte static "
                "scratch of csa2_select_topk_noalloc (use csa2_select_topk with a workspace)",
                Q, (long long)n_cols, need, csa2::SEL_SCRATCH_BYTES);
  void* ptr = nullptr;
  if (need > 0) {
    const hipError_t e = csa2::select_scratch(&ptr);
    if (e != hipSuccess)
      return fail(CSA2_EHIP, "csa2_select_topk_noalloc scratch lookup: %s", hipGetErrorString(e));
  }
  return hip_status(csa2::launch_select(scores, ld, Q, n_valid, col_ids, n_cols, k, 0, out, k,
                                        nullptr, 0, nullptr, ptr, (hipStream_t)stream),
                    "csa2_select_topk_noalloc launch");
}

csa2_status csa2_block_pool(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                            int64_t n_cols, int block, int n_blocks, int32_t* pool,
                            int64_t* pool_len, int k, int32_t* topk, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err[0] = 0;
  REQ(pool && pool_len, "pool and pool_len must not be NULL");
  REQ(k >= 0 && k <= n_blocks, "k=%d must be in [0, n_blocks=%d]", k, n_blocks);
  REQ(k == 0 || topk, "topk must not be NULL when k > 0");
  REQ(al(pool, 4) && al(pool_len, 8) && al0(topk, 4),
      "pool and topk must be 4-byte aligned, pool_len 8-byte aligned");
  if (block != 8) return fail(CSA2_EUNSUPPORTED, "block=%d: only blocks of 8 positions", block);
  const csa2_status st =
      select_common(scores, ld, Q, n_valid, nullptr, n_cols, n_blocks, ws, ws_bytes, 1);
  if (st != CSA2_OK) return st;
  return hip_status(csa2::launch_select(scores, ld, Q, n_valid, nullptr, n_cols, n_blocks, 1, pool,
                                        (int64_t)n_blocks * 8, pool_len, k, topk, ws,
                                        (hipStream_t)stream),
                    "csa2_block_pool launch");
}

static csa2_status select_attend_common(const float* scores, int64_t ld, int Q,
                                        const int64_t* n_valid, const int32_t* col_ids,
                                        int64_t n_cols, int k, int32_t* idx, int n_blocks,
                                        int32_t* pool, int64_t* pool_len, const uint16_t* q,
                                        const int32_t* q_seq, const csa2_cache* src,
                                        const uint8_t* swa_codes, const float* swa_scale,
                                        int64_t T_swa, const int64_t* swa_start,
                                        const int32_t* swa_len, float* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream, bool levels_ready) {
  REQ(scores && n_valid && idx && q && q_seq && out && swa_start && swa_len,
      "scores, n_valid, idx, q, q_seq, out, swa_start, swa_len must not be NULL");
  REQ(Q > 0 && Q < 256, "Q=%d must be in [1, 255] (larger batches: the separate calls)", Q);
  REQ(k >= 1 && k <= CSA2_MAX_K, "k=%d must be in [1, %d]", k, CSA2_MAX_K);
  REQ(n_blocks >= 0 && n_blocks <= CSA2_MAX_K, "n_blocks=%d must be in [0, %d]", n_blocks,
      CSA2_MAX_K);
  REQ(n_blocks == 0 || (pool && pool_len && !col_ids && k <= n_blocks),
      "with n_blocks > 0: pool and pool_len given, col_ids NULL, k <= n_blocks");
  REQ(n_cols >= 0 && n_cols <= CSA2_MAX_COLS, "n_cols=%lld must be in [0, %d]",
      (long long)n_cols, CSA2_MAX_COLS);
  REQ(ld >= n_cols && ld > 0, "ld=%lld < n_cols=%lld", (long long)ld, (long long)n_cols);
  const csa2_status cs = check_cache(src);
  if (cs != CSA2_OK) return cs;
  REQ(T_swa >= 0, "T_swa must be >= 0");
  REQ(T_swa == 0 || (swa_codes && swa_scale), "swa_codes / swa_scale NULL with T_swa > 0");
  REQ(al(q, 16) && al(out, 16) && al0(swa_codes, 16),
      "q, out and swa_codes must be 16-byte aligned");
  REQ(al(scores, 4) && al(n_valid, 8) && al0(col_ids, 4) && al(idx, 4) && al0(pool, 4) &&
          al0(pool_len, 8) && al(q_seq, 4) && al0(swa_scale, 4) && al(swa_start, 8) &&
          al(swa_len, 4) && al0(lse, 4),
      "n_valid, pool_len and swa_start must be 8-byte aligned, the other int32 / fp32 "
      "arrays 4-byte aligned");
  const int mode = n_blocks > 0 ? 1 : 0;
  const size_t need = csa2::select_attend_ws_bytes(Q, n_cols, mode, k);
  if (!ws || ws_bytes < need)
    return fail(CSA2_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0,
                need);
  REQ(al(ws, 256), "ws must be 256-byte aligned");
  if (device_checks())
    CHECKED(check_indices("q_seq", q_seq, 1, Q, nullptr, Q, 0,
                          src->batch > 0 ? src->batch : (int64_t)INT32_MAX, stream));
  return hip_status(csa2::launch_select_attend(scores, ld, Q, n_valid, col_ids, n_cols, mode,
                                               mode == 1 ? n_blocks : k, k, idx, pool, pool_len,
                                               q, q_seq, src->kv_codes, src->kv_scales, src->cap,
                                               swa_codes, swa_scale, T_swa, swa_start, swa_len,
                                               out, lse, ws, (hipStream_t)stream, levels_ready),
                    levels_ready ? "csa2_select_attend_levels launch" : "csa2_select_attend launch");
}

csa2_status csa2_select_attend(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                               const int32_t* col_ids, int64_t n_cols, int k, int32_t* idx,
                               int n_blocks, int32_t* pool, int64_t* pool_len, const uint16_t* q,
                               const int32_t* q_seq, const csa2_cache* src,
                               const uint8_t* swa_codes, const float* swa_scale, int64_t T_swa,
                               const int64_t* swa_start, const int32_t* swa_len, float* out,
                               float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return select_attend_common(scores, ld, Q, n_valid, col_ids, n_cols, k, idx, n_blocks, pool,
                              pool_len, q, q_seq, src, swa_codes, swa_scale, T_swa, swa_start,
                              swa_len, out, lse, ws, ws_bytes, stream, false);
}

csa2_status csa2_select_attend_levels(const float* scores, int64_t ld, int Q,
                                      const int64_t* n_valid, const int32_t* col_ids,
                                      int64_t n_cols, int k, int32_t* idx, int n_blocks,
                                      int32_t* pool, int64_t* pool_len, const uint16_t* q,
                                      const int32_t* q_seq, const csa2_cache* src,
                                      const uint8_t* swa_codes, const float* swa_scale,
                                      int64_t T_swa, const int64_t* swa_start,
                                      const int32_t* swa_len, float* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  REQ(!col_ids, "col_ids must be NULL (the levels are those of a full scan)");
  return select_attend_common(scores, ld, Q, n_valid, col_ids, n_cols, k, idx, n_blocks, pool,
                              pool_len, q, q_seq, src, swa_codes, swa_scale, T_swa, swa_start,
                              swa_len, out, lse, ws, ws_bytes, stream, true);
}

static csa2_status attend_common(const uint16_t* q, const int32_t* q_seq, int Q,
                                 const csa2_cache* src, const int32_t* idx, int k,
                                 const uint8_t* swa_codes, const float* swa_scale, int64_t T_swa,
                                 const int64_t* swa_start, const int32_t* swa_len, float* out,
                                 float* lse, void* ws, size_t ws_bytes,
                                 const csa2::RopeArgs& rp, void* stream) {
  REQ(q && q_seq && (out || rp.out_bf16) && swa_start && swa_len,
      "q, q_seq, out, swa_start, swa_len must not be NULL");
  const csa2_status cs = check_cache(src);
  if (cs != CSA2_OK) return cs;
  REQ(k >= 0 && k <= CSA2_MAX_K, "k=%d must be in [0, %d]", k, CSA2_MAX_K);
  REQ(k == 0 || idx, "idx must not be NULL when k > 0");
  REQ(T_swa >= 0, "T_swa must be >= 0");
  REQ(T_swa == 0 || (swa_codes && swa_scale), "swa_codes / swa_scale NULL with T_swa > 0");
  REQ(al(q, 16) && (!out || al(out, 16)) && (!rp.out_bf16 || al(rp.out_bf16, 16)) &&
          (!swa_codes || al(swa_codes, 16)),
      "q, out, swa_codes must be 16-byte aligned");
  REQ(al(q_seq, 4) && al0(idx, 4) && al0(swa_scale, 4) && al(swa_start, 8) && al(swa_len, 4) &&
          al0(lse, 4),
      "swa_start must be 8-byte aligned, q_seq, idx, swa_scale, swa_len, lse 4-byte aligned");
  REQ(!ws || al(ws, 16), "ws must be 16-byte aligned");
  REQ(Q > 0 && Q <= (1 << 24), "Q=%d must be in [1, 2^24]", Q);
  if (device_checks()) {
    CHECKED(check_indices("q_seq", q_seq, 1, Q, nullptr, Q, 0,
                          src->batch > 0 ? src->batch : (int64_t)INT32_MAX, stream));
    if (k > 0) CHECKED(check_indices("idx", idx, Q, k, nullptr, k, -1, src->cap, stream));
  }
  return hip_status(csa2::launch_attend(q, q_seq, Q, src->kv_codes, src->kv_scales, src->cap, idx,
                                        k, swa_codes, swa_scale, T_swa, swa_start, swa_len, out,
                                        lse, ws, ws_bytes, rp, (hipStream_t)stream),
                    rp.out_bf16 ? "csa2_sparse_attend_rope launch" : "csa2_sparse_attend launch");
}

csa2_status csa2_sparse_attend(const uint16_t* q, const int32_t* q_seq, int Q, const csa2_cache* src,
                               const int32_t* idx, int k, const uint8_t* swa_codes,
                               const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                               const int32_t* swa_len, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  REQ(out, "out must not be NULL");
  const csa2::RopeArgs none = {nullptr, 0, 0.f, nullptr, {}};
  return attend_common(q, q_seq, Q, src, idx, k, swa_codes, swa_scale, T_swa, swa_start, swa_len,
                       out, lse, ws, ws_bytes, none, stream);
}

csa2_status csa2_sparse_attend_rope(const uint16_t* q, const int32_t* q_seq, int Q,
                                    const csa2_cache* src, const int32_t* idx, int k,
                                    const uint8_t* swa_codes, const float* swa_scale,
                                    int64_t T_swa, const int64_t* swa_start,
                                    const int32_t* swa_len, const csa2_rope* rope,
                                    uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    void* stream) {
  g_err[0] = 0;
  REQ(rope && out, "rope and out must not be NULL");
  REQ(rope->dims >= 0 && rope->dims <= CSA2_MAX_ROPE && rope->dims % 2 == 0,
      "rope->dims=%d must be even and in [0, %d]", rope->dims, CSA2_MAX_ROPE);
  REQ(rope->dims == 0 || rope->q_pos, "rope->q_pos must not be NULL when rope->dims > 0");
  REQ(rope->dims == 0 || (rope->theta > 1.0f && rope->theta < INFINITY),
      "rope->theta must be finite and > 1");
  REQ(!rope->q_pos || al(rope->q_pos, 8), "rope->q_pos must be 8-byte aligned");
  csa2::RopeArgs rp = {rope->q_pos, rope->dims, rope->theta, out, {}};
  for (int i = 0; i < rope->dims / 2; ++i)
    rp.freq[i] = std::pow((double)rope->theta, -2.0 * (double)i / (double)rope->dims);
  return attend_common(q, q_seq, Q, src, idx, k, swa_codes, swa_scale, T_swa, swa_start, swa_len,
                       nullptr, lse, ws, ws_bytes, rp, stream);
}

size_t csa2_workspace_bytes(int op, int Q, int64_t n_cols, int k) {
  if (Q <= 0) return 0;
  switch (op) {
    case CSA2_OP_TOPK: return csa2::select_ws_bytes(Q, n_cols < 0 ? 0 : n_cols, 0);
    case CSA2_OP_POOL: return csa2::select_ws_bytes(Q, n_cols < 0 ? 0 : n_cols, 1);
    case CSA2_OP_ATTEND: return csa2::attend_ws_bytes(Q, k < 0 ? 0 : k);
    case CSA2_OP_SELECT_ATTEND:
    case CSA2_OP_POOL_ATTEND:
      if (k < 1) return 0;
      return csa2::select_attend_ws_bytes(Q, n_cols < 0 ? 0 : n_cols,
                                          op == CSA2_OP_POOL_ATTEND ? 1 : 0, k);
    default: return 0;
  }
}

int csa2_selftest(int32_t* counts, int n, void* stream) {
  const int c = csa2::selftest_count();
  if (!counts) return c;
  if (n < c) return -1;
  return csa2::launch_selftest(counts, (hipStream_t)stream) == hipSuccess ? 0 : -2;
}

}  // extern "C"
