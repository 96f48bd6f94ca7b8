// Steps a5 / a6 / a7 (selection): per-query top-k and the hierarchical
// block pool.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3.2 and Fig. 5: the first
// Full layer keeps its own top-512 and gives every block of 8 positions the
// maximum score among them, keeps the 2048 best blocks (16,384 positions)
// as the pool that Reindex layers search.  Ordering used everywhere:
// (score desc, id asc).
//
// The selection itself (maxima pyramid, slot-major keep-best-kk rounds,
// one query's whole selection) is in select_core.h; this file holds the
// maxima kernel, the selection kernel and their host launchers.
#include "common.h"
#include "launch.h"
#include "select_core.h"

#include <mutex>

namespace csa2 {

// ------------------------------------------------------------ maxima
// One workgroup per (query, 4096 columns): levels 1..4 of that span.  With
// spec (few queries) a thread's 16 scores are requested before n_valid
// arrives, when they lie within the launch's columns.
__global__ __launch_bounds__(256) void k_maxima(const float* __restrict__ scores, int64_t ld,
                                                const int64_t* __restrict__ n_valid,
                                                int64_t n_cols, int64_t nchunk, LevelDesc d,
                                                uint32_t* __restrict__ ws, int vec, int spec) {
  __shared__ uint32_t wmax[4];
  const int q = (int)(gridDim.x / nchunk - 1 - blockIdx.x / nchunk);   // last queries first
  const int64_t chunk = blockIdx.x % nchunk;
  const int tid = threadIdx.x;
  const int64_t c0 = chunk * 4096 + (int64_t)tid * 16;
  const float* sp = scores + (int64_t)q * ld;
  const bool pre = spec && vec && c0 + 16 <= n_cols;
  f32x4_t v0 = {}, v1 = {}, v2 = {}, v3 = {};
  if (pre) {
    const f32x4_t* vp = (const f32x4_t*)(sp + c0);
    v0 = vp[0]; v1 = vp[1]; v2 = vp[2]; v3 = vp[3];
  }
  const int64_t n0 = n_valid[q];
  const int64_t n = n0 < n_cols ? n0 : n_cols;
  if (chunk * 4096 >= n) return;
  uint32_t k1a = 0, k1b = 0;
  if (vec && c0 + 16 <= n) {
    if (!pre) {
      const f32x4_t* vp = (const f32x4_t*)(sp + c0);
      v0 = vp[0]; v1 = vp[1]; v2 = vp[2]; v3 = vp[3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k1a = max(k1a, max(f32_key(v0[i]), f32_key(v1[i])));
      k1b = max(k1b, max(f32_key(v2[i]), f32_key(v3[i])));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (c0 + i < n) k1a = max(k1a, f32_key(sp[c0 + i]));
      if (c0 + 8 + i < n) k1b = max(k1b, f32_key(sp[c0 + 8 + i]));
    }
  }
  const int64_t g1 = c0 / 8;
  const int64_t G1 = groups_at(n, 1);
  uint32_t* l1 = ws + d.off[1] + (int64_t)q * d.stride[1];
  if (g1 < G1) l1[g1] = k1a;
  if (g1 + 1 < G1) l1[g1 + 1] = k1b;
  if (d.nlev < 2) return;
  uint32_t k = max(k1a, k1b);
  k = max(k, __shfl_xor(k, 1));
  k = max(k, __shfl_xor(k, 2));
  if ((tid & 3) == 0) {
    const int64_t g = chunk * 64 + tid / 4;
    if (g < groups_at(n, 2)) ws[d.off[2] + (int64_t)q * d.stride[2] + g] = k;
  }
  if (d.nlev < 3) return;
  k = max(k, __shfl_xor(k, 4));
  k = max(k, __shfl_xor(k, 8));
  k = max(k, __shfl_xor(k, 16));
  if ((tid & 31) == 0) {
    const int64_t g = chunk * 8 + tid / 32;
    if (g < groups_at(n, 3)) ws[d.off[3] + (int64_t)q * d.stride[3] + g] = k;
  }
  if (d.nlev < 4) return;
  k = max(k, __shfl_xor(k, 32));
  if ((tid & 63) == 0) wmax[tid >> 6] = k;
  __syncthreads();
  if (tid == 0) {
    const uint32_t m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (chunk < groups_at(n, 4)) ws[d.off[4] + (int64_t)q * d.stride[4] + chunk] = m;
  }
}

// ------------------------------------------------------------ select
// One workgroup per query.  The 256-thread selector runs many queries per
// CU (prefill): five waves per SIMD keep five workgroups resident.
template <int NT, int PER>
__global__ __launch_bounds__(NT, (NT <= 256 ? 5 : 1)) void k_select(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, LevelDesc d,
    const uint32_t* __restrict__ ws, int kk, int mode, int32_t* __restrict__ out, int64_t out_ld,
    int64_t* __restrict__ out_len, int k2, int32_t* __restrict__ out2, int vec_out, int spec) {
  __shared__ SelShared<NT> sh;
  const int q = gridDim.x - 1 - blockIdx.x;        // last queries (most columns when causal) first
  (void)select_query<NT, PER>(q, scores, ld, n_valid, col_ids, n_cols, d, ws, kk, mode, out,
                              out_ld, out_len, k2, out2, vec_out, spec, true, sh);
}

// ------------------------------------------------------------ scratch
// Static scratch of the allocation-free top-k entry point: the maxima
// pyramid lives here instead of in a caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends; its address is
// looked up once per device (the host-side name is only a stand-in and must
// never be passed to a kernel).  Nothing in it has to start at zero: the
// maxima kernel writes every group a selection reads.
static __device__ __align__(256) uint8_t scratch[SEL_SCRATCH_BYTES];

namespace {
constexpr int SEL_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SEL_MAX_DEVICES] = {};
}  // namespace

hipError_t select_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SEL_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------ host side
static LevelDesc make_levels(int Q, int64_t n_cols, int mode) {
  LevelDesc d = {};
  int L = 0;
  while (groups_at(n_cols, L) > SEL_CAP) ++L;
  if (L < mode) L = mode;
  d.nlev = L;
  int64_t off = 0;
  for (int l = 1; l <= L; ++l) {
    d.off[l] = off;
    d.stride[l] = (groups_at(n_cols, l) + 15) / 16 * 16; // 64-byte aligned rows
    off += (int64_t)Q * d.stride[l];
  }
  return d;
}

size_t select_ws_bytes(int Q, int64_t n_cols, int mode) {
  const LevelDesc d = make_levels(Q, n_cols, mode);
  size_t words = 0;
  for (int l = 1; l <= d.nlev; ++l) words += (size_t)Q * (size_t)d.stride[l];
  return words * 4;
}

LevelDesc select_levels(int Q, int64_t n_cols, int mode) { return make_levels(Q, n_cols, mode); }

hipError_t launch_maxima(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         int64_t n_cols, const LevelDesc& d, uint32_t* ws, hipStream_t stream) {
  const int64_t nchunk = (n_cols + 4095) / 4096;
  const bool al16 = ((uintptr_t)scores & 15) == 0;
  const int vec_max = (ld % 4 == 0) && al16;    // 16-byte row starts
  const int spec = Q <= 64;                      // first loads ahead of n_valid
  if (d.nlev > 0 && nchunk > 0)
    hipLaunchKernelGGL(k_maxima, dim3((unsigned)(nchunk * Q)), dim3(256), 0, stream, scores, ld,
                       n_valid, n_cols, nchunk, d, ws, vec_max, spec);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         const int32_t* col_ids, int64_t n_cols, int kk, int mode, int32_t* out,
                         int64_t out_ld, int64_t* out_len, int k2, int32_t* out2, void* ws,
                         hipStream_t stream, bool levels_ready) {
  const LevelDesc d = make_levels(Q, n_cols, mode);
  const int vec_out = ((uintptr_t)out & 15) == 0 && out_ld % 4 == 0;   // 16-byte output rows
  const int spec = Q <= 64;                      // first loads ahead of n_valid
  if (!levels_ready) launch_maxima(scores, ld, Q, n_valid, n_cols, d, (uint32_t*)ws, stream);
  // one round over at most 4096 candidates: 256-thread workgroups, several per CU
  if (mode == 0 && n_cols <= 256 * SEL_PER) {
    hipLaunchKernelGGL((k_select<256, SEL_PER>), dim3((unsigned)Q), dim3(256), 0, stream, scores, ld, n_valid,
                       col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld, out_len, k2,
                       out2, vec_out, spec);
  } else
    hipLaunchKernelGGL((k_select<SEL_NT, SEL_CAP / SEL_NT>), dim3((unsigned)Q), dim3(SEL_NT), 0, stream, scores, ld,
                       n_valid, col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld,
                       out_len, k2, out2, vec_out, spec);
  return hipGetLastError();
}

}  // namespace csa2
