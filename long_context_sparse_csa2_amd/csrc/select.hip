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
                                                uint32_t* __restrict__ ws, int vec) {
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
  if (vec && c0 + 16 <= n) {
    const f32x4_t* vp = (const f32x4_t*)(sp + c0);
    const f32x4_t v0 = vp[0], v1 = vp[1], v2 = vp[2], v3 = vp[3];
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

// Candidates of one selection live in registers: slot i of thread t holds
// candidate e = i * 1024 + t (valid iff e < cnt), so candidate order is
// (slot, thread) order and every LDS access below is conflict-free.
constexpr int SEL_PER = SEL_CAP / SEL_THREADS;     // 16 slots per thread
constexpr int SEL_SMALL = 256;

// number of register slots that hold candidates (uniform over the block)
__device__ __forceinline__ int used_slots(int cnt) { return (cnt + SEL_THREADS - 1) / SEL_THREADS; }

// Threshold of the best kk of the cnt candidates (cnt > kk >= 1).
//
// Search on the key interval [lo, hi] that holds the kk-th best key: each
// pass bins the keys inside it by (key - lo) >> s, with s chosen so that at
// most 2048 bins cover the interval, keeps the bin holding the krem-th best
// key and shrinks the interval to it.  Once the interval holds at most
// SEL_SMALL candidates their exact kk-th key is found by ranking them
// against each other.  Result: keys above hi are in, keys inside [lo, hi]
// are in for the first `tie_lim` of them in candidate (= id) order, keys
// below lo are out.
__device__ __forceinline__ void threshold_search(const uint32_t (&kr)[SEL_PER], int cnt, int kk, uint32_t* hist,
                                 uint32_t* red, uint32_t* bc, uint32_t* small, uint32_t& lo_out,
                                 uint32_t& hi_out, uint32_t& tie_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int ns = used_slots(cnt);
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if (i >= ns) break;
    if (i * SEL_THREADS + tid < cnt) {
      mn = min(mn, kr[i]);
      mx = max(mx, kr[i]);
    }
  }
  block_minmax(mn, mx, red);

  uint32_t lo = mn, hi = mx;
  uint32_t krem = (uint32_t)kk;
  uint32_t incnt = (uint32_t)cnt;          // candidates with key in [lo, hi]
  uint32_t tie_lim;
  while (true) {
    if (lo == hi) { tie_lim = krem; break; }
    if (incnt <= (uint32_t)SEL_SMALL) {
      // gather the interval's keys and rank them exactly
      if (tid == 0) bc[3] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < SEL_PER; ++i) {
        if (i >= ns) break;
        const uint32_t k = kr[i];
        if (i * SEL_THREADS + tid < cnt && k >= lo && k <= hi) small[atomicAdd(&bc[3], 1u)] = k;
      }
      __syncthreads();
      if (tid < (int)incnt) {
        const uint32_t mine = small[tid];
        uint32_t gt = 0, ge = 0;
        for (uint32_t j = 0; j < incnt; ++j) {
          const uint32_t o = small[j];
          gt += o > mine;
          ge += o >= mine;
        }
        if (gt < krem && ge >= krem) { bc[0] = mine; bc[1] = gt; }
      }
      __syncthreads();
      const uint32_t t = bc[0], g = bc[1];
      __syncthreads();
      lo = hi = t;
      tie_lim = krem - g;
      break;
    }
    const uint32_t span = hi - lo;                                   // range - 1
    const int bits = 32 - __clz(span);
    const int sh = bits > 11 ? bits - 11 : 0;
    hist[tid] = 0u;
    hist[tid + SEL_THREADS] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i) {
      if (i >= ns) break;
      const uint32_t k = kr[i];
      const bool in = i * SEL_THREADS + tid < cnt && k >= lo && k <= hi;
      const uint32_t bin = (k - lo) >> sh;
      // lanes of a wave that share one bin (concentrated scores) add once
      const uint64_t act = __ballot(in);
      if (act) {
        const int first = __ffsll((long long)act) - 1;
        const uint32_t b0 = __builtin_amdgcn_readlane(bin, first);
        const uint64_t same = __ballot(in && bin == b0);
        if (same == act) {
          if (lane == first) atomicAdd(&hist[b0], (uint32_t)__popcll(act));
        } else if (in) {
          atomicAdd(&hist[bin], 1u);
        }
      }
    }
    __syncthreads();
    // thread t owns bins 2047-2t (hi) and 2046-2t (lo); counts from the top
    const int bh = 2047 - 2 * tid, bl = bh - 1;
    const uint32_t hh = hist[bh], hl = hist[bl];
    const uint32_t incl = block_incl_scan(hh + hl, red);
    const uint32_t excl = incl - hh - hl;
    if (excl < krem && incl >= krem) {
      if (excl + hh >= krem) { bc[0] = (uint32_t)bh; bc[1] = excl; bc[2] = hh; }
      else { bc[0] = (uint32_t)bl; bc[1] = excl + hh; bc[2] = hl; }
    }
    __syncthreads();
    const uint32_t d = bc[0], above = bc[1], inbin = bc[2];
    __syncthreads();
    krem -= above;
    const uint32_t nlo = lo + (d << sh);
    const uint32_t top = (d << sh) + ((1u << sh) - 1u);
    const uint32_t nhi = top >= span ? hi : lo + top;
    lo = nlo;
    hi = nhi;
    incnt = inbin;
    if (inbin == krem) { tie_lim = krem; break; }                    // the whole bin is in
  }
  lo_out = lo;
  hi_out = hi;
  tie_out = tie_lim;
}

// Write the ids of the selected candidates (all of them if sel_all) to
// sel[0..) in candidate order; returns how many.  table holds 2 x 256 words.
__device__ __forceinline__ int compact_ids(const uint32_t (&kr)[SEL_PER], const uint32_t (&ir)[SEL_PER], int cnt,
                           bool sel_all, uint32_t lo, uint32_t hi, uint32_t tie_lim,
                           uint32_t* sel, uint32_t* table, uint32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the masks are recomputed in the second pass rather than kept (SGPR budget)
  const int ns = used_slots(cnt);
  if (tid < 256) table[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if (i >= ns) break;
    const bool v = i * SEL_THREADS + tid < cnt;
    const uint64_t gm = __ballot(v && (sel_all || kr[i] > hi));
    const uint64_t tm = __ballot(v && !sel_all && kr[i] >= lo && kr[i] <= hi);
    if (lane == 0) table[i * 16 + wave] = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(tm) << 16);
  }
  __syncthreads();
  // exclusive scan over the 256 (slot, wave) counts in candidate order
  const uint32_t v = tid < 256 ? table[tid] : 0u;
  const uint32_t incl = block_incl_scan(v, red);
  if (tid < 256) table[256 + tid] = incl - v;
  if (tid == 255) red[31] = incl;
  __syncthreads();
  const uint32_t total = red[31];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if (i >= ns) break;
    const bool v2 = i * SEL_THREADS + tid < cnt;
    const bool g = v2 && (sel_all || kr[i] > hi);
    const bool t = v2 && !sel_all && kr[i] >= lo && kr[i] <= hi;
    const uint64_t gm = __ballot(g);
    const uint64_t tm = __ballot(t);
    const uint32_t pre = table[256 + i * 16 + wave];
    const uint32_t gb = (pre & 0xFFFFu) + (uint32_t)__popcll(gm & below);
    const uint32_t tb = (pre >> 16) + (uint32_t)__popcll(tm & below);
    if (g || (t && tb < tie_lim)) sel[gb + min(tb, tie_lim)] = ir[i];
  }
  __syncthreads();
  const uint32_t ng = total & 0xFFFFu, nt = total >> 16;
  return (int)(ng + min(nt, tie_lim));
}

// ------------------------------------------------------------ select
// mode 0: top-kk columns -> out[q][0..kk) ids (col_ids mapped), -1 padded.
// mode 1: best kk blocks of 8 -> out[q][0..8kk) positions, out_len[q]; then,
//         if k2 > 0, the top-k2 positions inside that pool -> out2[q][0..k2).
//         (With k2 <= kk the top-k2 of all columns lies inside the pool.)
__global__ __launch_bounds__(SEL_THREADS) void k_select(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, LevelDesc d,
    const uint32_t* __restrict__ ws, int kk, int mode, int32_t* __restrict__ out, int64_t out_ld,
    int64_t* __restrict__ out_len, int k2, int32_t* __restrict__ out2) {
  __shared__ uint32_t sel[SEL_KK_MAX];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t small[SEL_SMALL];
  __shared__ uint32_t table[512];
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
    if (mode == 1) {
      if (tid == 0) out_len[q] = 0;
      for (int i = tid; i < k2; i += SEL_THREADS) out2[(int64_t)q * k2 + i] = -1;
    }
    return;
  }
  auto level_key = [&](int lvl, int64_t g) __attribute__((always_inline)) -> uint32_t {
    return lvl == 0 ? f32_key(srow[g]) : ws[d.off[lvl] + (int64_t)q * d.stride[lvl] + g];
  };
  uint32_t kr[SEL_PER], ir[SEL_PER];
  // candidates of level lvl: all its groups (first == true) or the children
  // of the cnt groups listed in sel[] (ascending)
  auto load = [&](int lvl, bool first, int pcnt) __attribute__((always_inline)) -> int {
    int c;
    if (first) {
      c = (int)groups_at(n, lvl);
    } else {
      const int64_t gc = groups_at(n, lvl);
      const int64_t rem = gc - 8 * (int64_t)sel[pcnt - 1];
      c = 8 * (pcnt - 1) + (rem < 8 ? (int)rem : 8);
    }
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i) {
      if (i >= used_slots(c)) break;
      const int e = i * SEL_THREADS + tid;
      uint32_t id = 0, key = 0;
      if (e < c) {
        id = first ? (uint32_t)e : sel[e >> 3] * 8u + (uint32_t)(e & 7);
        key = level_key(lvl, id);
      }
      kr[i] = key;
      ir[i] = id;
    }
    __syncthreads();                      // sel[] may be overwritten after this
    return c;
  };
  // keep the best `want` of the loaded candidates in sel[] (ids ascending)
  auto keep = [&](int c, int want) __attribute__((always_inline)) -> int {
    uint32_t lo = 0, hi = 0, tl = 0;
    const bool all = c <= want;
    if (!all) threshold_search(kr, c, want, hist, red, bc, small, lo, hi, tl);
    return compact_ids(kr, ir, c, all, lo, hi, tl, sel, table, red);
  };

  int lvl = 0;
  while (groups_at(n, lvl) > SEL_CAP) ++lvl;
  if (lvl < stop) lvl = stop;
  int cnt = load(lvl, true, 0);
  while (true) {
    cnt = keep(cnt, kk);
    if (lvl == stop) break;
    --lvl;
    cnt = load(lvl, false, cnt);
  }

  if (mode == 0) {
    for (int i = tid; i < kk; i += SEL_THREADS) {
      int32_t v = -1;
      if (i < cnt) v = col_ids ? col_ids[(int64_t)q * ld + sel[i]] : (int32_t)sel[i];
      orow[i] = v;
    }
    return;
  }
  for (int i = tid; i < kk * 8; i += SEL_THREADS) {
    int32_t v = -1;
    if (i < cnt * 8) {
      const int64_t p = (int64_t)sel[i >> 3] * 8 + (i & 7);
      if (p < n) v = (int32_t)p;
    }
    orow[i] = v;
  }
  if (tid == 0) {
    const int64_t rem = n - 8 * (int64_t)sel[cnt - 1];
    out_len[q] = (int64_t)8 * (cnt - 1) + (rem < 8 ? rem : 8);
  }
  if (k2 > 0) {                          // the Full layer's own top-k, from inside its pool
    cnt = load(0, false, cnt);
    cnt = keep(cnt, k2);
    for (int i = tid; i < k2; i += SEL_THREADS)
      out2[(int64_t)q * k2 + i] = i < cnt ? (int32_t)sel[i] : -1;
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
                         int64_t out_ld, int64_t* out_len, int k2, int32_t* out2, void* ws,
                         hipStream_t stream) {
  const LevelDesc d = make_levels(Q, n_cols, mode);
  const int64_t nchunk = (n_cols + 4095) / 4096;
  if (d.nlev > 0 && nchunk > 0) {
    const int vec = (ld % 4 == 0) && (((uintptr_t)scores & 15) == 0);   // 16-byte row starts
    hipLaunchKernelGGL(k_maxima, dim3((unsigned)(nchunk * Q)), dim3(256), 0, stream, scores, ld,
                       n_valid, n_cols, nchunk, d, (uint32_t*)ws, vec);
  }
  hipLaunchKernelGGL(k_select, dim3((unsigned)Q), dim3(SEL_THREADS), 0, stream, scores, ld,
                     n_valid, col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld,
                     out_len, k2, out2);
  return hipGetLastError();
}

}  // namespace csa2
