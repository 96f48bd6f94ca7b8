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

// ------------------------------------------------------------ select
// One workgroup of NT threads (1024, or 256 for small rounds) per query.
// The candidates of one round (at most SEL_CAP, in id order) live in
// registers, thread-major: thread t holds candidates 16t .. 16t + 15 (in the
// first round 16 consecutive groups, later the 8 children of parents 2t and
// 2t + 1), so the order-preserving compaction is one block scan of
// per-thread counts.
//
// Floor.  A round keeps its best kk parents; each kept parent's maximum
// child has the parent's key, so when the next round wants at most as many
// as were kept, its answer lies among the children whose key is at least
// the smallest kept key (the floor) and the children below it are dropped
// before the threshold search.
constexpr int SEL_PER = 16;                        // candidates per thread
constexpr int SEL_SMALL = 64;                      // intervals this small are ranked exactly
constexpr int SEL_BINS = 2048;

template <int NT>
struct SelShared {
  uint32_t lists[2][SEL_KK_MAX];      // parent ids of this round / ids it keeps
  uint32_t hist[SEL_BINS];
  uint32_t small[SEL_SMALL];
  uint32_t red[2][(NT / 64)];
  uint32_t mm[2][(NT / 64)];
  uint32_t cn[2][(NT / 64)];
  uint32_t bc[4][4];
};

// Inclusive block-wide sum; `total` gets the block total.  red must not be
// reused by the caller until after the next barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < (NT / 64); ++w) {
    const uint32_t x = red[w];
    pre += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  return incl + pre;
}

// Bit i set iff candidate i is considered and its key lies in [lo, hi].
template <int PER>
__device__ __forceinline__ uint32_t range_mask(const uint32_t (&kr)[PER], uint32_t cmask,
                                               uint32_t lo, uint32_t hi) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) m |= (kr[i] >= lo && kr[i] <= hi) ? (1u << i) : 0u;
  return m & cmask;
}

// Threshold of the best kk of the m considered candidates (m > kk >= 1),
// given their min and max keys; cmask = this thread's considered ones.
//
// Search on the key interval [lo, hi] that holds the kk-th best key: each
// pass bins the keys inside it by (key - lo) >> s, with s chosen so that at
// most 2048 bins cover the interval, keeps the bin holding the krem-th best
// key and shrinks the interval to it.  Once the interval holds at most
// SEL_SMALL candidates their exact kk-th key is found by ranking them
// against each other.  Result: keys above hi are in, keys inside [lo, hi]
// are in for the first `tie_lim` of them in candidate (= id) order, keys
// below lo are out.  The histogram must be zero on entry and is left zero;
// so is the gather counter sh.bc[3][3].
template <int NT, int PER>
__device__ __forceinline__ void threshold_search(const uint32_t (&kr)[PER], uint32_t cmask,
                                                 int m, int kk, uint32_t mn, uint32_t mx,
                                                 SelShared<NT>& sh, uint32_t& lo_out,
                                                 uint32_t& hi_out, uint32_t& tie_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t lo = mn, hi = mx;
  uint32_t krem = (uint32_t)kk;
  uint32_t incnt = (uint32_t)m;            // considered candidates with key in [lo, hi]
  uint32_t tie_lim;
  int pass = 0;
  while (true) {
    if (lo == hi) { tie_lim = krem; break; }
    const uint32_t imask = range_mask<PER>(kr, cmask, lo, hi);
    if (incnt <= (uint32_t)SEL_SMALL) {
      // gather the interval's keys: wave prefix of per-thread counts, one
      // LDS atomic per wave for the wave's base
      const uint32_t c = (uint32_t)__popc(imask);
      const uint32_t incl = wave_incl_sum(c);
      uint32_t base = 0;
      if (lane == 63) base = atomicAdd(&sh.bc[3][3], incl);
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63);
      uint32_t pos = base + incl - c;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((imask >> i) & 1u) sh.small[pos++] = kr[i];
      __syncthreads();
      // rank each gathered key against all of them, RS threads per key
      constexpr int RS = NT / SEL_SMALL;
      const int ci = tid / RS, part = tid % RS;
      const uint32_t mine = ci < (int)incnt ? sh.small[ci] : 0u;
      uint32_t gt = 0, ge = 0;
      for (uint32_t j = part; j < incnt; j += RS) {
        const uint32_t o = sh.small[j];
        gt += o > mine;
        ge += o >= mine;
      }
#pragma unroll
      for (int off = 1; off < RS; off <<= 1) { gt += __shfl_xor(gt, off); ge += __shfl_xor(ge, off); }
      if (part == 0 && ci < (int)incnt && gt < krem && ge >= krem) { sh.bc[2][0] = mine; sh.bc[2][1] = gt; }
      __syncthreads();
      const uint32_t t = sh.bc[2][0], g = sh.bc[2][1];
      if (tid == 0) sh.bc[3][3] = 0u;     // gather counter; next used after further barriers
      lo = hi = t;
      tie_lim = krem - g;
      break;
    }
    const uint32_t span = hi - lo;                                   // range - 1
    const int bits = 32 - __clz(span);
    const int shf = bits > 11 ? bits - 11 : 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((imask >> i) & 1u) atomicAdd(&sh.hist[(kr[i] - lo) >> shf], 1u);
    __syncthreads();
    // thread t owns (SEL_BINS / NT) consecutive bins from the top, counted downwards
    uint32_t hb[(SEL_BINS / NT)];
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < (SEL_BINS / NT); ++j) {
      hb[j] = sh.hist[SEL_BINS - 1 - (SEL_BINS / NT) * tid - j];
      sh.hist[SEL_BINS - 1 - (SEL_BINS / NT) * tid - j] = 0u;                  // leave it zero
      v += hb[j];
    }
    uint32_t tot;
    const uint32_t incl = block_scan<NT>(v, sh.red[pass & 1], tot);
    uint32_t* bcp = sh.bc[pass & 1];
    if (incl - v < krem && incl >= krem) {
      uint32_t acc = incl - v;
#pragma unroll
      for (int j = 0; j < (SEL_BINS / NT); ++j) {
        if (acc < krem && acc + hb[j] >= krem) {
          bcp[0] = (uint32_t)(SEL_BINS - 1 - (SEL_BINS / NT) * tid - j);
          bcp[1] = acc;
          bcp[2] = hb[j];
        }
        acc += hb[j];
      }
    }
    __syncthreads();
    const uint32_t d = bcp[0], above = bcp[1], inbin = bcp[2];
    ++pass;
    krem -= above;
    const uint32_t nlo = lo + (d << shf);
    const uint32_t top = (d << shf) + ((1u << shf) - 1u);
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

// One keep-best-`want` round over the candidates this thread holds in
// kr[0 .. nv) (thread-major: ids increase with the thread, then the slot):
// candidates below floor_key are dropped, the threshold of the rest found
// and the kept ids written in id order to `keep` (id_of(i) is slot i's id).
// rb picks the reduction buffers (alternate it between rounds).  Ends with a
// barrier; returns the kept count, the threshold interval's low end and the
// smallest considered key (the next round's floor), and whether every
// considered candidate was kept.
struct RoundOut {
  int kept;
  uint32_t lo, mn;
  bool all;
};

template <int NT, int PER, typename IdOf>
__device__ __forceinline__ RoundOut select_round(const uint32_t (&kr)[PER], int nv, uint32_t floor_key,
                                                 int want, SelShared<NT>& sh, int rb, uint32_t* keep,
                                                 IdOf id_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t cmask = 0, mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool c = i < nv && kr[i] >= floor_key;
    cmask |= c ? (1u << i) : 0u;
    mn = c ? min(mn, kr[i]) : mn;
    mx = c ? max(mx, kr[i]) : mx;
  }
  mn = wave_min_all(mn);
  mx = wave_max_all(mx);
  const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum((uint32_t)__popc(cmask)), 63);
  if (lane == 0) { sh.red[rb][wave] = mn; sh.mm[rb][wave] = mx; sh.cn[rb][wave] = wc; }
  __syncthreads();
  int m = 0;
#pragma unroll
  for (int w = 0; w < (NT / 64); ++w) {
    mn = min(mn, sh.red[rb][w]);
    mx = max(mx, sh.mm[rb][w]);
    m += (int)sh.cn[rb][w];
  }
  uint32_t lo = 0, hi = 0, tl = 0;
  const bool all = m <= want;
  if (!all) threshold_search<NT, PER>(kr, cmask, m, want, mn, mx, sh, lo, hi, tl);
  uint32_t gm = cmask, tm = 0;
  if (!all) {
    gm = hi == 0xFFFFFFFFu ? 0u : range_mask<PER>(kr, cmask, hi + 1u, 0xFFFFFFFFu);
    tm = range_mask<PER>(kr, cmask, lo, hi);
  }
  const uint32_t ngt = (uint32_t)__popc(gm), ntie = (uint32_t)__popc(tm);
  const uint32_t packed = ngt | (ntie << 16);           // both sums stay below 2^16
  uint32_t tot;
  const uint32_t excl = block_scan<NT>(packed, sh.red[rb ^ 1], tot) - packed;
  const uint32_t gt_before = excl & 0xFFFFu, tie_before = excl >> 16;
  // this thread's ties in id order while the tie limit lasts
  uint32_t take = tl > tie_before ? tl - tie_before : 0u;
  uint32_t tk = 0, trest = tm;
  while (take > 0 && trest != 0) {
    tk |= trest & (0u - trest);
    trest &= trest - 1u;
    --take;
  }
  const uint32_t km = gm | tk;
  uint32_t pos = gt_before + min(tie_before, tl);
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if ((km >> i) & 1u) keep[pos++] = id_of(i);
  const int kept = all ? m : (int)((tot & 0xFFFFu) + min(tot >> 16, tl));
  __syncthreads();
  return RoundOut{kept, lo, mn, all};
}

// Raw words of 8 consecutive entries b .. b+7 of a level array or a score
// row into raw[off .. off + 8).  vec: the 8 words lie inside the row and
// start 16-byte aligned (two vector loads); otherwise word j is read at
// min(b + j, len - 1) and the caller masks the ones at or past len.
__device__ __forceinline__ void load_run8(const uint32_t* src, int64_t b, int64_t len, bool vec,
                                          uint32_t (&raw)[SEL_PER], int off) {
  if (vec) {
    const u32x4_t x0 = *(const u32x4_t*)(src + b);
    const u32x4_t x1 = *(const u32x4_t*)(src + b + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { raw[off + j] = x0[j]; raw[off + 4 + j] = x1[j]; }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) raw[off + j] = src[b + j < len ? b + j : len - 1];
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, LevelDesc d,
    const uint32_t* __restrict__ ws, int kk, int mode, int32_t* __restrict__ out, int64_t out_ld,
    int64_t* __restrict__ out_len, int k2, int32_t* __restrict__ out2, int vec0) {
  __shared__ SelShared<NT> sh;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n0 = n_valid[q];
  const int64_t n = n0 < 0 ? 0 : (n0 < n_cols ? n0 : n_cols);
  const float* srow = scores + (int64_t)q * ld;
  int32_t* orow = out + (int64_t)q * out_ld;
  const int stop = mode;
  const int64_t out_w = mode == 0 ? kk : (int64_t)kk * 8;

  if (n == 0) {
    for (int64_t i = tid; i < out_w; i += NT) orow[i] = -1;
    if (mode == 1) {
      if (tid == 0) out_len[q] = 0;
      for (int i = tid; i < k2; i += NT) out2[(int64_t)q * k2 + i] = -1;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < (SEL_BINS / NT); ++j) sh.hist[(SEL_BINS / NT) * tid + j] = 0u;
  if (tid == 0) sh.bc[3][3] = 0u;

  int cur = 0;                      // sh.lists[cur]: parents of the round being loaded
  int lvl = 0;
  while (groups_at(n, lvl) > (int64_t)NT * SEL_PER) ++lvl;
  if (lvl < stop) lvl = stop;
  bool first = true;
  int pcnt = 0;
  int rb = 0;                       // alternates the reduction buffers between rounds
  uint32_t floor_key = 0;           // children below it cannot be in this round's answer

  while (true) {
    // ---- candidates of level lvl (thread t: 16t .. 16t+15), every load in flight at once
    const uint32_t* par = sh.lists[cur];
    const int64_t gl = groups_at(n, lvl);
    int cnt;
    if (first) {
      cnt = (int)gl;
    } else {
      const int64_t rem = gl - 8 * (int64_t)par[pcnt - 1];
      cnt = 8 * (pcnt - 1) + (rem < 8 ? (int)rem : 8);
    }
    const int e0 = SEL_PER * tid;
    const int nv = cnt - e0 < 0 ? 0 : (cnt - e0 > SEL_PER ? SEL_PER : cnt - e0);
    const bool is_score = lvl == 0;
    const uint32_t* src = is_score ? (const uint32_t*)srow
                                   : ws + d.off[lvl] + (int64_t)q * d.stride[lvl];
    const bool vok = !is_score || vec0;              // level rows are padded to 16 words
    uint32_t kr[SEL_PER];
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i) kr[i] = 0u;
    uint32_t p0 = 0, p1 = 0;
    if (nv > 0) {
      int64_t b0 = e0, b1 = e0 + 8;
      if (!first) {
        // candidates 16t .. 16t+15 are the children of parents 2t and 2t+1
        p0 = par[e0 >> 3];
        p1 = nv > 8 ? par[(e0 >> 3) + 1] : p0;
        b0 = (int64_t)p0 * 8;
        b1 = (int64_t)p1 * 8;
      }
      load_run8(src, b0, gl, vok, kr, 0);
      load_run8(src, b1, gl, vok, kr, 8);
      if (is_score) {
#pragma unroll
        for (int i = 0; i < SEL_PER; ++i) kr[i] = f32_key(__uint_as_float(kr[i]));
      }
    }
    const int want = (lvl == 0 && mode == 1) ? k2 : kk;
    const RoundOut ro = select_round<NT, SEL_PER>(
        kr, nv, floor_key, want, sh, rb, sh.lists[cur ^ 1], [&](int i) __attribute__((always_inline)) {
          return first ? (uint32_t)(e0 + i) : (i < 8 ? p0 : p1) * 8u + (uint32_t)(i & 7);
        });
    const int kept = ro.kept;
    cur ^= 1;
    rb ^= 1;
    first = false;
    pcnt = kept;
    const uint32_t* sel = sh.lists[cur];
    const bool map_cols = lvl == stop && mode == 0 && col_ids;

    if (lvl == stop && mode == 0) {
      for (int i = tid; i < kk; i += NT) {
        int32_t o = -1;
        if (i < kept) o = map_cols ? col_ids[(int64_t)q * ld + sel[i]] : (int32_t)sel[i];
        orow[i] = o;
      }
      return;
    }
    if (lvl == 1 && mode == 1) {           // the pool: positions of the kept blocks
      for (int i = tid; i < kk * 8; i += NT) {
        int32_t o = -1;
        if (i < kept * 8) {
          const int64_t p = (int64_t)sel[i >> 3] * 8 + (i & 7);
          if (p < n) o = (int32_t)p;
        }
        orow[i] = o;
      }
      if (tid == 0) {
        const int64_t rem = n - 8 * (int64_t)sel[kept - 1];
        out_len[q] = (int64_t)8 * (kept - 1) + (rem < 8 ? rem : 8);
      }
      if (k2 <= 0) return;
    }
    if (lvl == 0 && mode == 1) {           // the Full layer's own top-k, from inside its pool
      for (int i = tid; i < k2; i += NT)
        out2[(int64_t)q * k2 + i] = i < kept ? (int32_t)sel[i] : -1;
      return;
    }
    --lvl;
    const int want_next = (lvl == 0 && mode == 1) ? k2 : kk;
    floor_key = kept >= want_next ? (ro.all ? ro.mn : ro.lo) : 0u;
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

hipError_t launch_select(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         const int32_t* col_ids, int64_t n_cols, int kk, int mode, int32_t* out,
                         int64_t out_ld, int64_t* out_len, int k2, int32_t* out2, void* ws,
                         hipStream_t stream) {
  const LevelDesc d = make_levels(Q, n_cols, mode);
  const int64_t nchunk = (n_cols + 4095) / 4096;
  const bool al16 = ((uintptr_t)scores & 15) == 0;
  const int vec_max = (ld % 4 == 0) && al16;    // 16-byte row starts
  const int vec = (ld % 16 == 0) && al16;       // every run of 8 / 16 scores inside its row
  if (d.nlev > 0 && nchunk > 0) {
    hipLaunchKernelGGL(k_maxima, dim3((unsigned)(nchunk * Q)), dim3(256), 0, stream, scores, ld,
                       n_valid, n_cols, nchunk, d, (uint32_t*)ws, vec_max);
  }
  // one round over at most 4096 candidates: 256-thread workgroups, several per CU
  if (mode == 0 && n_cols <= 256 * SEL_PER) {
    hipLaunchKernelGGL(k_select<256>, dim3((unsigned)Q), dim3(256), 0, stream, scores, ld, n_valid,
                       col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld, out_len, k2,
                       out2, vec);
  } else
    hipLaunchKernelGGL(k_select<1024>, dim3((unsigned)Q), dim3(1024), 0, stream, scores, ld,
                       n_valid, col_ids, n_cols, d, (const uint32_t*)ws, kk, mode, out, out_ld,
                       out_len, k2, out2, vec);
  return hipGetLastError();
}

}  // namespace csa2
