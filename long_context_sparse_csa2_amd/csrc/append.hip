// Decode-time append: the per-sequence state block of the V4 KV layout
// ("DeepSeek-V4" page, Fig. 6: a fixed-size block per request holding the
// SWA entries of the most recent tokens and the uncompressed tail that is
// not yet ready for compression).
//
// One decode token per sequence.  The compressor (k_compress_quant in its
// append mode) first turns a group of m tokens that the new token completes
// into a cache entry; this kernel then files the token: its raw latent and
// compression logits go to tail slot n_tok mod m (unless it completed the
// group), its SWA latent is quantised to one FP8 row (E4M3FN codes, one fp32
// scale sigma = max|x| / 448) in ring slot n_tok mod W, the geometry the
// sequence's next query sees is written, and the count advances.
#include "common.h"
#include "launch.h"

namespace csa2 {

// One wave per sequence; lane l owns channels 8l .. 8l + 7.
__global__ __launch_bounds__(64) void k_append_state(
    const uint16_t* __restrict__ h_new, const uint16_t* __restrict__ z_new,
    const uint16_t* __restrict__ swa_new, int m, uint16_t* __restrict__ tail_h,
    uint16_t* __restrict__ tail_z, int64_t* __restrict__ n_tok, uint8_t* __restrict__ swa_codes,
    float* __restrict__ swa_scale, int64_t W, int64_t* __restrict__ n_vis,
    int64_t* __restrict__ swa_start, int32_t* __restrict__ swa_len) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int64_t t = n_tok[b];                         // every lane reads before lane 0 writes
  const int s = (int)(t % m);
  if (s < m - 1) {                                    // the group is not complete: keep the token
    const int64_t src = (int64_t)b * D_LAT + lane * 8;
    const int64_t dst = ((int64_t)b * (m - 1) + s) * D_LAT + lane * 8;
    *(u32x4_t*)(tail_h + dst) = *(const u32x4_t*)(h_new + src);
    *(u32x4_t*)(tail_z + dst) = *(const u32x4_t*)(z_new + src);
  }
  if (W > 0) {
    const u32x4_t v = *(const u32x4_t*)(swa_new + (int64_t)b * D_LAT + lane * 8);
    float x[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[2 * c] = __uint_as_float(v[c] << 16);
      x[2 * c + 1] = __uint_as_float(v[c] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(x[c]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sig = amax / 448.0f;                  // IEEE division, as every quotient here
    uint32_t lo = 0, hi = 0;
    if (sig > 0.f) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float q = x[c] / sig;
        const uint32_t code = e4m3_encode_pos(fabsf(q)) | (q < 0.f ? 0x80u : 0u);
        if (c < 4) lo |= code << (8 * c); else hi |= code << (8 * (c - 4));
      }
    }
    const int64_t slot = (int64_t)b * W + t % W;
    *(uint2*)(swa_codes + slot * D_LAT + lane * 8) = make_uint2(lo, hi);
    if (lane == 0) swa_scale[slot] = sig;
  }
  if (lane == 0) {
    const int64_t n = t + 1;
    const int64_t len = n < W ? n : W;
    if (n_vis) n_vis[b] = n / m;
    if (swa_start) swa_start[b] = W > 0 ? (n - len) % W : 0;
    if (swa_len) swa_len[b] = (int32_t)len;
    n_tok[b] = n;
  }
}

hipError_t launch_append_state(const uint16_t* h_new, const uint16_t* z_new,
                               const uint16_t* swa_new, int B, int m, uint16_t* tail_h,
                               uint16_t* tail_z, int64_t* n_tok, uint8_t* swa_codes,
                               float* swa_scale, int64_t W, int64_t* n_vis, int64_t* swa_start,
                               int32_t* swa_len, hipStream_t stream) {
  hipLaunchKernelGGL(k_append_state, dim3((unsigned)B), dim3(64), 0, stream, h_new, z_new, swa_new,
                     m, tail_h, tail_z, n_tok, swa_codes, swa_scale, W, n_vis, swa_start, swa_len);
  return hipGetLastError();
}

}  // namespace csa2
