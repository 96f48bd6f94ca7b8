// Steps a5 / a6 / a7 (selection): per-query top-k and the hierarchical
// block pool.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3.2 and Fig. 5: the first
// Full layer keeps its own top-512 and gives every block of 8 positions the
// maximum score among them, keeps the 2048 best blocks (16,384 positions)
// as the pool that Reindex layers search.  Ordering used everywhere:
// (score desc, id asc).
//
// Design.  Both selections run on 8-way maxima pyramids: level 0 is the
// scores, level l + 1 holds the maximum of 8 consecutive level-l values.
// With the same ordering at every level, the best kk groups of a level are
// contained in the children of the best kk groups of the level above (a
// child ranks below its parent's rank, and a group whose parent ranks
// below kk has kk groups above it whose maxima beat or tie it with lower
// ids).  So a query's selection starts at the first level with at most
// 16,384 groups, which one workgroup holds in LDS, keeps the best kk there,
// expands them into their 8 children each (at most 16,384), keeps the best
// kk of those, and so on down to the scores (top-k) or to the blocks of 8
// (pool).  Each keep-best-kk is an exact MSB-first radix select in LDS on
// order-preserving uint32 keys, starting below the bits all candidates
// share, followed by an order-preserving compaction; ties at the threshold
// go to the lowest ids because the candidates are kept in id order.  Only
// integer histograms and scans are used, so the result is deterministic.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_KK_MAX = 2048;

struct LevelDesc {
  int64_t off[SEL_MAX_LEVELS + 1];      // uint32 offset of level l (l >= 1) in the workspace
  int64_t stride[SEL_MAX_LEVELS + 1];   // per-query length of level l
  int nlev;                             // levels 1..nlev are present
};

// ------------------------------------------------------------ maxima
// One workgroup per (query, 4096 columns): levels 1..4 of that span.
__global__ __launch_bounds__(256) void k_maxima(const float* __restrict__ scores, int64_t ld,
                                                const int64_t* __restrict__ n_valid,
                                                int64_t n_cols, int64_t nchunk, LevelDesc d,
                                                uint32_t* __restrict__ ws) {
  __shared__ uint32_t wmax[4];
  const int q = (int)(blockIdx.x / nchunk);
  const int64_t chunk = blockIdx.x % nchunk;
  const int64_t n0 = n_valid[q];
  const int64_t n = n0 < n_cols ? n0 : n_cols;
  if (chunk * 4096 >= n) return;
  const int tid = threadIdx.x;
  const int64_t c0 = chunk * 4096 + (int64_t)tid * 16;
  const float* sp = scores + (int64_t)q * ld;
  uint32_t k1a = 0, k1b = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (c0 + i < n) k1a = max(k1a, f32_key(sp[c0 + i]));
    if (c0 + 8 + i < n) k1b = max(k1b, f32_key(sp[c0 + 8 + i]));
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

// ------------------------------------------------------ block helpers
// Inclusive scan of one value per thread over the 1024-thread block.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) red[wave] = v;
  __syncthreads();
  uint32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += red[w];
  __syncthreads();
  return v + pre;
}

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, __shfl_xor(mn, off));
    mx = max(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) { red[wave] = mn; red[16 + wave] = mx; }
  __syncthreads();
  mn = red[0];
  mx = red[16];
  for (int w = 1; w < SEL_THREADS / 64; ++w) { mn = min(mn, red[w]); mx = max(mx, red[16 + w]); }
  __syncthreads();
}

// Keep the best kk of cnt candidates (keys[i], ids[i]) in place, in id
// order.  Requires cnt > kk >= 1 and ascending ids.
__device__ void block_keep_best(uint32_t* keys, uint32_t* ids, int cnt, int kk, uint32_t* hist,
                                uint32_t* red, uint32_t* bc) {
  const int tid = threadIdx.x;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = tid; i < cnt; i += SEL_THREADS) {
    const uint32_t k = keys[i];
    mn = min(mn, k);
    mx = max(mx, k);
  }
  block_minmax(mn, mx, red);

  // threshold search: after it, candidates whose masked key exceeds
  // `prefix` are in, those equal to it are ties (the first `krem` of them in
  // id order are in, all of them if tie_all), the rest are out.
  uint32_t prefix, mask;
  uint32_t krem = (uint32_t)kk;
  bool tie_all = false;
  const uint32_t diff = mn ^ mx;
  if (diff == 0u) {
    prefix = mn;
    mask = 0xFFFFFFFFu;
  } else {
    int shift = 32 - __clz(diff);
    mask = shift == 32 ? 0u : (0xFFFFFFFFu << shift);
    prefix = mx & mask;
    while (shift > 0) {
      const int db = shift < 11 ? shift : 11;
      shift -= db;
      const uint32_t dmask = (1u << db) - 1u;
      for (int i = tid; i < 2048; i += SEL_THREADS) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < cnt; i += SEL_THREADS) {
        const uint32_t k = keys[i];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      // thread t owns bins 2047-2t (hi) and 2046-2t (lo); counts from the top
      const int hi = 2047 - 2 * tid, lo = hi - 1;
      const uint32_t hh = hist[hi], hl = hist[lo];
      const uint32_t incl = block_incl_scan(hh + hl, red);
      const uint32_t excl = incl - hh - hl;
      if (excl < krem && incl >= krem) {
        if (excl + hh >= krem) { bc[0] = (uint32_t)hi; bc[1] = excl; bc[2] = hh; }
        else { bc[0] = (uint32_t)lo; bc[1] = excl + hh; bc[2] = hl; }
      }
      __syncthreads();
      const uint32_t dsel = bc[0], above = bc[1], inbin = bc[2];
      __syncthreads();
      krem -= above;
      prefix |= dsel << shift;
      mask |= dmask << shift;
      if (inbin == krem) { tie_all = true; break; }
    }
  }

  // order-preserving compaction: thread t owns [t*per, t*per + per)
  const int per = (cnt + SEL_THREADS - 1) / SEL_THREADS;   // <= 16
  const int beg = tid * per;
  uint32_t kr[16], ir[16];
  uint32_t ngt = 0, ntie = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = beg + i;
    kr[i] = 0u; ir[i] = 0u;
    if (i < per && x < cnt) {
      kr[i] = keys[x];
      ir[i] = ids[x];
      const uint32_t mk = kr[i] & mask;
      ngt += mk > prefix;
      ntie += mk == prefix;
    }
  }
  const uint32_t packed = ngt | (ntie << 16);           // both sums stay below 2^16
  const uint32_t excl = block_incl_scan(packed, red) - packed;
  const uint32_t tie_lim = tie_all ? 0xFFFFFFFFu : krem;
  const uint32_t gt_before = excl & 0xFFFFu, tie_before = excl >> 16;
  uint32_t pos = gt_before + min(tie_before, tie_lim);
  uint32_t tr = tie_before;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = beg + i;
    if (i < per && x < cnt) {
      const uint32_t mk = kr[i] & mask;
      const bool tie = mk == prefix;
      const bool sel = mk > prefix || (tie && tr < tie_lim);
      tr += tie;
      if (sel) { keys[pos] = kr[i]; ids[pos] = ir[i]; ++pos; }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------ select
// mode 0: top-kk columns -> out[q][0..kk) ids (col_ids mapped), -1 padded.
// mode 1: best kk blocks of 8 -> out[q][0..8kk) positions, out_len[q].
__global__ __launch_bounds__(SEL_THREADS) void k_select(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, LevelDesc d,
    const uint32_t* __restrict__ ws, int kk, int mode, int32_t* __restrict__ out, int64_t out_ld,
    int64_t* __restrict__ out_len) {
  __shared__ uint32_t keys[SEL_CAP];
  __shared__ uint32_t ids[SEL_CAP];
  __shared__ uint32_t tmp[SEL_KK_MAX];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t red[32];
  __shared__ uint32_t bc[4];

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n0 = n_valid[q];
  const int64_t n = n0 < 0 ? 0 : (n0 < n_cols ? n0 : n_cols);
  const float* srow = scores + (int64_t)q * ld;
  int32_t* orow = out + (int64_t)q * out_ld;
  const int stop = mode;
  const int64_t out_w = mode == 0 ? kk : (int64_t)kk * 8;

  if (n == 0) {
    for (int64_t i = tid; i < out_w; i += SEL_THREADS) orow[i] = -1;
    if (mode == 1 && tid == 0) out_len[q] = 0;
    return;
  }
  auto level_key = [&](int lvl, int64_t g) -> uint32_t {
    return lvl == 0 ? f32_key(srow[g]) : ws[d.off[lvl] + (int64_t)q * d.stride[lvl] + g];
  };

  int lvl = 0;
  while (groups_at(n, lvl) > SEL_CAP) ++lvl;
  if (lvl < stop) lvl = stop;
  int cnt = (int)groups_at(n, lvl);
  for (int i = tid; i < cnt; i += SEL_THREADS) {
    keys[i] = level_key(lvl, i);
    ids[i] = (uint32_t)i;
  }
  __syncthreads();

  while (true) {
    if (cnt > kk) {
      block_keep_best(keys, ids, cnt, kk, hist, red, bc);
      cnt = kk;
    }
    if (lvl == stop) break;
    // expand the kept groups into their children one level down
    for (int i = tid; i < cnt; i += SEL_THREADS) tmp[i] = ids[i];
    __syncthreads();
    const int64_t gc = groups_at(n, lvl - 1);
    const int64_t last = tmp[cnt - 1];
    const int64_t rem = gc - 8 * last;
    const int lastc = rem < 8 ? (int)rem : 8;
    const int ncnt = 8 * (cnt - 1) + lastc;
    for (int i = tid; i < ncnt; i += SEL_THREADS) {
      const uint32_t child = tmp[i >> 3] * 8u + (uint32_t)(i & 7);
      ids[i] = child;
      keys[i] = level_key(lvl - 1, child);
    }
    __syncthreads();
    cnt = ncnt;
    --lvl;
  }

  if (mode == 0) {
    for (int i = tid; i < kk; i += SEL_THREADS) {
      int32_t v = -1;
      if (i < cnt) v = col_ids ? col_ids[(int64_t)q * ld + ids[i]] : (int32_t)ids[i];
      orow[i] = v;
    }
  } else {
    for (int i = tid; i < kk * 8; i += SEL_THREADS) {
      int32_t v = -1;
      if (i < cnt * 8) {
        const int64_t p = (int64_t)ids[i >> 3] * 8 + (i & 7);
        if (p < n) v = (int32_t)p;
      }
      orow[i] = v;
    }
    if (tid == 0) {
      const int64_t rem = n - 8 * (int64_t)ids[cnt - 1];
      out_len[q] = (int64_t)8 * (cnt - 1) + (rem < 8 ? rem : 8);
    }
  }
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
    d.stride[l] = groups_at(n_cols, l);
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

hipError_t launch_select(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         const int32_t* col_ids, int64_t n_cols, int kk, int mode, int32_t* out,
                         int64_t out_ld, int64_t* out_len, void* ws, hipStream_t stream) {
  const LevelDesc d = make_levels(Q, n_cols, mode);
  const int64_t nchunk = (n_cols + 4095) / 4096;
  if (d.nlev > 0 && nchunk > 0) {
    hipLaunchKernelGGL(k_maxima, dim3((unsigned)(nchunk * Q)), dim3(256), 0, stream, scores, ld,
                       n_valid, n_cols, nchunk, d, (uint32_t*)ws);
  }
  hipLaunchKernelGGL(k_select, dim3((unsigned)Q), dim3(SEL_THREADS), 0, stream, scores, ld,
                     n_valid, col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld,
                     out_len);
  return hipGetLastError();
}

}  // namespace csa2
