// Selection machinery shared by the top-k / pool kernel and the fused
// selection + attention kernel: 8-way maxima pyramid levels, the slot-major
// keep-best-kk round and one query's whole selection.
//
// Report digest "DeepSeek-V4.1-Flash", section 2.3.2 and Fig. 5: the first
// Full layer keeps its own top-512 and gives every block of 8 positions the
// maximum score among them, keeps the 2048 best blocks (16,384 positions)
// as the pool that Reindex layers search.  Ordering used everywhere:
// (score desc, id asc).
//
// Both selections run on 8-way maxima pyramids: level 0 is the scores,
// level l + 1 holds the maximum of 8 consecutive level-l values.  With the
// same ordering at every level, the best kk groups of a level are contained
// in the children of the best kk groups of the level above (a child ranks
// below its parent's rank, and a group whose parent ranks below kk has kk
// groups above it whose maxima beat or tie it with lower ids).  So a
// query's selection starts at the first level with at most 16,384 groups,
// which one workgroup holds in registers, keeps the best kk there, expands
// them into their 8 children each (at most 16,384), keeps the best kk of
// those, and so on down to the scores (top-k) or to the blocks of 8 (pool).
// Each keep-best-kk is an exact MSB-first radix select in LDS on
// order-preserving uint32 keys, starting below the bits all candidates
// share, followed by an order-preserving compaction; ties at the threshold
// go to the lowest ids because the candidates are kept in id order.  Only
// integer histograms and scans are used, so the result is deterministic.
#pragma once

#include "common.h"

namespace csa2 {

constexpr int SEL_KK_MAX = 2048;

struct LevelDesc {
  int64_t off[SEL_MAX_LEVELS + 1];      // uint32 offset of level l (l >= 1) in the workspace
  int64_t stride[SEL_MAX_LEVELS + 1];   // per-query length of level l
  int nlev;                             // levels 1..nlev are present
};

// ------------------------------------------------------------ select
// One workgroup of NT threads (1024, or 256 for small rounds) per query.
// The candidates of one round (PER slots per lane, at most NT * PER, in id
// order) live in registers slot-major: slot i of lane l in wave w holds
// candidate c = 64 PER w + 64 i + l, with key 0 for "no candidate" (no fp32
// value maps to key 0).  The candidates of one slot across a wave are then
// consecutive, so an order-preserving compaction is a ballot and a masked
// bit count per slot, and the only block-wide step is a prefix over per-wave
// totals.  A round's block-wide bookkeeping (histogram scans) runs in one
// wave while the others wait at the barrier.
//
// Floor.  A round keeps its best kk parents; each kept parent's maximum
// child has the parent's key, so when the next round wants at most as many
// as were kept, its answer lies among the children whose key is at least
// the smallest kept key (the floor).  That round searches its threshold
// between the floor and the best parent's key: those bounds are known, so it
// needs no min / max pass, and children below the floor keep their keys but
// fall outside the bounds, so neither the histogram nor the compaction
// counts them.
constexpr int SEL_PER = 16;                        // candidate slots per lane (small rounds)
#ifndef SEL_NT
#define SEL_NT 1024                                // threads of the 16,384-candidate selector
#endif
constexpr int SEL_SMALL = 64;                      // intervals this small are ranked exactly
constexpr int SEL_BINS = 2048;

template <int NT>
struct SelShared {
  uint32_t lists[2][SEL_KK_MAX + 64]; // parent ids of this round / ids it keeps (+ 64 spare slots)
  uint32_t hist[SEL_BINS + 64];        // + one dummy bin per lane for keys outside the interval
  uint32_t small[SEL_SMALL];
  uint32_t wred[3][NT / 64];          // per-wave min, max, count
  uint32_t wcnt[NT / 64];             // per-wave kept counts (above | ties << 16)
  uint32_t bc[2][4];                  // histogram pass results, alternating
  uint32_t sres[3];                   // small interval: threshold, keys above it, keys equal
  uint32_t gather;                    // small-interval gather counter
};

// Number of set bits of m below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave 0's scan of the histogram, from the top bin down: lane l sums bins
// [SEL_BINS - 32 (l + 1), SEL_BINS - 32 l) in groups of 4, the lane whose
// range holds the krem-th best key finds its group and re-reads it to find
// the bin, and every lane then zeroes its bins.  out = (bin, keys above it,
// keys in it, total).
__device__ __forceinline__ void hist_scan(uint32_t* hist, uint32_t krem, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int base = SEL_BINS - 32 * (lane + 1);
  uint32_t g[8], s = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const u32x4_t x = *(const u32x4_t*)&hist[base + 4 * v];
    g[v] = x[0] + x[1] + x[2] + x[3];
    s += g[v];
  }
  const uint32_t incl = wave_incl_sum(s);
  const uint32_t excl = incl - s;
  if (lane == 63) out[3] = incl;
  if (excl < krem && incl >= krem) {
    uint32_t acc = excl, gv = 0, gacc = 0;
#pragma unroll
    for (int v = 7; v >= 0; --v) {
      if (acc < krem && acc + g[v] >= krem) { gv = (uint32_t)v; gacc = acc; }
      acc += g[v];
    }
    const u32x4_t bb = *(const u32x4_t*)&hist[base + 4 * gv];
    acc = gacc;
    uint32_t bin = 0, above = 0, inbin = 0;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (acc < krem && acc + bb[j] >= krem) { bin = 4 * gv + (uint32_t)j; above = acc; inbin = bb[j]; }
      acc += bb[j];
    }
    out[0] = (uint32_t)base + bin;
    out[1] = above;
    out[2] = inbin;
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) *(u32x4_t*)&hist[base + 4 * v] = u32x4_t{0u, 0u, 0u, 0u};
}

// One keep-best-`want` round over the candidates in kr (slot-major, key 0 =
// none).  known: every candidate's key lies in [kmn, kmx] (kmn >= 1) and the
// min / max / count pass is skipped.  The kept ids go to `keep` in id order
// (id_of(i) is slot i's id).  Ends with a barrier; returns the kept count,
// the low end of the threshold interval, bounds of the considered keys, and
// whether every considered candidate was kept.
struct RoundOut {
  int kept;
  uint32_t lo, mn, mx;
  bool all;
};

template <int NT, int PER, typename IdOf>
__device__ __forceinline__ RoundOut select_round(const uint32_t (&kr)[PER], bool known,
                                                 uint32_t kmn, uint32_t kmx, int want,
                                                 SelShared<NT>& sh, uint32_t* keep, IdOf id_of) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t mn = kmn, mx = kmx;
  uint32_t m = 0xFFFFFFFFu;                       // considered count (unknown when known)
  if (!known) {
    uint32_t mnm1 = 0xFFFFFFFFu, mxx = 0u, cnt = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mnm1 = min(mnm1, kr[i] - 1u);               // key 0 wraps to the top
      mxx = max(mxx, kr[i]);
      cnt += kr[i] != 0u ? 1u : 0u;
    }
    mnm1 = wave_min_all(mnm1);
    mxx = wave_max_all(mxx);
    cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(cnt), 63);
    if (lane == 0) { sh.wred[0][wave] = mnm1; sh.wred[1][wave] = mxx; sh.wred[2][wave] = cnt; }
    __syncthreads();
    uint32_t a = 0xFFFFFFFFu, b = 0u, c = 0u;
    if (lane < NW) { a = sh.wred[0][lane]; b = sh.wred[1][lane]; c = sh.wred[2][lane]; }
    mn = wave_min_all(a) + 1u;
    mx = wave_max_all(b);
    m = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(c), 63);
  }
  bool all = m <= (uint32_t)want;
  uint32_t lo = mn, hi = mx, tl = 0;
  bool ties_all = true;                 // every key in [lo, hi] is kept
  if (!all) {
    uint32_t krem = (uint32_t)want;
    uint32_t incnt = m;                           // candidates with key in [lo, hi]
    int pass = 0;
    while (true) {
      if (lo == hi) { tl = krem; ties_all = incnt == krem; break; }
      const uint32_t span = hi - lo;
      if (incnt <= (uint32_t)SEL_SMALL) {
        // gather the interval's keys (any order); a slot holding some takes
        // its place with one LDS atomic
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const bool in = kr[i] - lo <= span;
          const uint64_t mk = __ballot(in);
          if (mk) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&sh.gather, (uint32_t)__popcll(mk));
            base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
            if (in) sh.small[base + lanes_below(mk)] = kr[i];
          }
        }
        __syncthreads();
        // rank each gathered key against all of them, RS threads per key
        constexpr int RS = NT / SEL_SMALL;
        const int ci = tid / RS, part = tid % RS;
        const uint32_t mine = ci < (int)incnt ? sh.small[ci] : 0u;
        uint32_t cnt = 0;                         // keys above mine | keys >= mine << 16
#pragma unroll
        for (int it = 0; it < SEL_SMALL / RS; ++it) {
          const int j = part + it * RS;
          const uint32_t o = sh.small[j];
          cnt += j < (int)incnt ? (o > mine ? 1u : 0u) + (o >= mine ? 0x10000u : 0u) : 0u;
        }
#pragma unroll
        for (int off = 1; off < RS; off <<= 1) cnt += (uint32_t)__shfl_xor((int)cnt, off);
        const uint32_t gt = cnt & 0xFFFFu, ge = cnt >> 16;
        if (part == 0 && ci < (int)incnt && gt < krem && ge >= krem) {
          sh.sres[0] = mine;
          sh.sres[1] = gt;
          sh.sres[2] = ge - gt;
        }
        __syncthreads();
        const uint32_t t = sh.sres[0], g = sh.sres[1], eq = sh.sres[2];
        if (tid == 0) sh.gather = 0u;             // next used after further barriers
        lo = hi = t;
        tl = krem - g;
        ties_all = eq == tl;
        break;
      }
      const int bits = 32 - __clz(span);
      const int shf = bits > 11 ? bits - 11 : 0;
      if (pass == 0) {
        // every candidate lies in [lo, hi]; key 0 (none) goes to the lane's
        // own dummy bin (one shared dummy would serialise the atomics)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const uint32_t d = kr[i] - lo;
          atomicAdd(&sh.hist[d <= span ? d >> shf : (uint32_t)(SEL_BINS + lane)], 1u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const uint32_t d = kr[i] - lo;
          if (d <= span) atomicAdd(&sh.hist[d >> shf], 1u);
        }
      }
      __syncthreads();
      uint32_t* bcp = sh.bc[pass & 1];
      if (wave == 0) hist_scan(sh.hist, krem, bcp);
      __syncthreads();
      const uint32_t total = bcp[3];
      ++pass;
      if (total <= krem) { all = true; break; }   // first pass of a known round: all fit
      const uint32_t d = bcp[0], above = bcp[1], inbin = bcp[2];
      krem -= above;
      const uint32_t nlo = lo + (d << shf);
      const uint32_t top = (d << shf) + ((1u << shf) - 1u);
      const uint32_t nhi = top >= span ? hi : lo + top;
      lo = nlo;
      hi = nhi;
      incnt = inbin;
      if (inbin == krem) { tl = krem; break; }    // the whole bin is in (ties_all)
    }
  }
  // ---- order-preserving compaction.  Usually every key in [lo, hi] is in
  // (the whole bin, or no tie straddles the k-th key) and the kept keys are
  // those >= lo; otherwise the keys above hi and the first tl keys inside
  // [lo, hi] in id order.
  const uint32_t span = hi - lo;
  const bool fast = all || ties_all;
  uint32_t ngt = 0, ntie = 0;
  if (fast) {
#pragma unroll
    for (int i = 0; i < PER; ++i) ngt += (uint32_t)__popcll(__ballot(kr[i] >= lo));
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      ngt += (uint32_t)__popcll(__ballot(kr[i] > hi));
      ntie += (uint32_t)__popcll(__ballot(kr[i] - lo <= span));
    }
  }
  if (lane == 0) sh.wcnt[wave] = ngt | (ntie << 16);    // both stay below 2^16
  __syncthreads();
  const uint32_t incl = wave_incl_sum(lane < NW ? sh.wcnt[lane] : 0u);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)incl, wave - 1) : 0u;
  const uint32_t gt_before = before & 0xFFFFu, tie_before = before >> 16;
  if (fast) {
    uint32_t pos = gt_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = kr[i] >= lo;                  // lo >= 1: key 0 is never in
      const uint64_t km = __ballot(in);
      const uint32_t at = in ? pos + lanes_below(km) : (uint32_t)(SEL_KK_MAX + lane);  // spare
      keep[at] = id_of(i);
      pos += (uint32_t)__popcll(km);
    }
  } else {
    uint32_t take = tl > tie_before ? tl - tie_before : 0u;
    uint32_t pos = gt_before + min(tie_before, tl);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool tie = kr[i] - lo <= span;
      const uint64_t tm = __ballot(tie);
      const uint32_t nt = (uint32_t)__popcll(tm);
      bool tk = tie;
      if (nt > take) tk = tie && lanes_below(tm) < take;
      take = nt > take ? 0u : take - nt;
      const bool in = kr[i] > hi || tk;
      const uint64_t km = __ballot(in);
      if (km) {
        if (in) keep[pos + lanes_below(km)] = id_of(i);
        pos += (uint32_t)__popcll(km);
      }
    }
  }
  const int kept = fast ? (int)(tot & 0xFFFFu) : (int)((tot & 0xFFFFu) + min(tot >> 16, tl));
  __syncthreads();
  return RoundOut{kept, lo, mn, mx, all};
}

// One query's selection (the body of k_select): the kept columns end in
// LDS, ascending.  With `write` the outputs go to global memory (top-k ids
// mapped through col_ids, or the pool, its length and the top-k of mode 1);
// without it nothing is written.  Returns the final list: for mode 0 the
// top-kk columns, for mode 1 the top-k2 entries (or, with k2 == 0, the
// kept blocks); `identity` marks the case where every valid column is kept
// (ids 0..kept-1, list unused).  Must be called by all NT threads.
struct SelResult {
  int kept;
  bool identity;
  const uint32_t* list;
};

template <int NT, int PER>
__device__ __forceinline__ SelResult select_query(
    int q, const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ n_valid,
    const int32_t* __restrict__ col_ids, int64_t n_cols, const LevelDesc& d,
    const uint32_t* __restrict__ ws, int kk, int mode, int32_t* __restrict__ out, int64_t out_ld,
    int64_t* __restrict__ out_len, int k2, int32_t* __restrict__ out2, int vec_out, int spec,
    bool write, SelShared<NT>& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = scores + (int64_t)q * ld;
  int32_t* orow = out + (int64_t)q * out_ld;
  const int stop = mode;
  const int64_t out_w = mode == 0 ? kk : (int64_t)kk * 8;
  const int cap = NT * PER;
  const int cbase = 64 * PER * wave + lane;          // candidate of slot 0

  // spec (few queries, latency-bound): the first round's loads go out before
  // n_valid arrives, at the level n_cols gives, every index clamped into the
  // level's row; otherwise (many queries: causal prefill rows hold fewer
  // valid columns than n_cols) they wait for n_valid and stop at the valid
  // groups
  auto level_of = [&](int64_t n) {
    int l = 0;
    while (groups_at(n, l) > (int64_t)cap) ++l;
    return l < stop ? stop : l;
  };
  auto src_of = [&](int l) {
    return l == 0 ? (const uint32_t*)srow : ws + d.off[l] + (int64_t)q * d.stride[l];
  };
  int lvl = level_of(n_cols);
  uint32_t kr[PER];
  auto load_first = [&](int l, int64_t nn) {
    const uint32_t* src = src_of(l);
    const int64_t len64 = groups_at(nn, l);
    const int last = (int)(len64 < cap ? len64 : cap) - 1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = cbase + 64 * i;
      kr[i] = src[c < last ? c : last];
    }
  };
  if (spec && n_cols > 0) load_first(lvl, n_cols);
  const int64_t n0 = n_valid[q];
  const int64_t n = n0 < 0 ? 0 : (n0 < n_cols ? n0 : n_cols);
  if (n == 0) {
    if (write) {
      for (int64_t i = tid; i < out_w; i += NT) orow[i] = -1;
      if (mode == 1) {
        if (tid == 0) out_len[q] = 0;
        for (int i = tid; i < k2; i += NT) out2[(int64_t)q * k2 + i] = -1;
      }
    }
    return SelResult{0, true, nullptr};
  }
  if (mode == 0 && n <= kk) {              // every valid column is kept, in id order
    if (write) {
      for (int i = tid; i < kk; i += NT) {
        int32_t o = -1;
        if (i < n) o = col_ids ? col_ids[(int64_t)q * ld + i] : i;
        orow[i] = o;
      }
    }
    return SelResult{(int)n, true, nullptr};
  }
  {
    const int ln = level_of(n);
    if (!spec || ln != lvl) { lvl = ln; load_first(lvl, n); }
  }
#pragma unroll
  for (int j = 0; j < (SEL_BINS / NT); ++j) sh.hist[(SEL_BINS / NT) * tid + j] = 0u;
  if (tid == 0) sh.gather = 0u;

  // pool output: positions of the kept blocks (sel, ascending) and its length
  auto write_pool = [&](int kept, const uint32_t* sel) __attribute__((always_inline)) {
    if (vec_out) {                       // one block's 8 positions as two 16-byte stores
      for (int b = tid; b < kk; b += NT) {
        const int64_t base = b < kept ? (int64_t)sel[b] * 8 : n;
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = base + j < n ? (uint32_t)(base + j) : 0xFFFFFFFFu;
        *(u32x4_t*)(orow + 8 * b) = u32x4_t{o[0], o[1], o[2], o[3]};
        *(u32x4_t*)(orow + 8 * b + 4) = u32x4_t{o[4], o[5], o[6], o[7]};
      }
    } else {
      for (int i = tid; i < kk * 8; i += NT) {
        int32_t o = -1;
        if (i < kept * 8) {
          const int64_t p = (int64_t)sel[i >> 3] * 8 + (i & 7);
          if (p < n) o = (int32_t)p;
        }
        orow[i] = o;
      }
    }
    if (tid == 0) {
      const int64_t rem = n - 8 * (int64_t)sel[kept - 1];
      out_len[q] = (int64_t)8 * (kept - 1) + (rem < 8 ? rem : 8);
    }
  };
  bool pool_pending = false;
  int cur = 0;                      // sh.lists[cur]: parents of the round being loaded
  bool first = true;
  int pcnt = 0;
  uint32_t floor_key = 0;           // children below it cannot be in this round's answer
  uint32_t top_key = 0;             // the best key of the previous round
  uint32_t pid[PER];            // child rounds: parent id of each slot

  while (true) {
    const int gl = (int)groups_at(n, lvl);            // n <= 2^26 fits
    const bool is_score = lvl == 0;
    if (first) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t k = is_score ? f32_key(__uint_as_float(kr[i])) : kr[i];
        kr[i] = cbase + 64 * i < gl ? k : 0u;
      }
    } else {
      // slot i of this lane: child (lane & 7) of parent (c >> 3) in the kept
      // list; pid = ~0 marks a slot without a child
      const uint32_t* par = sh.lists[cur];
      const uint32_t* src = src_of(lvl);
#pragma unroll
      for (int i = 0; i < PER; ++i) {    // every parent read first, then every load
        const int p = (cbase + 64 * i) >> 3;
        pid[i] = par[p < pcnt ? p : 0];
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int p = (cbase + 64 * i) >> 3;
        const uint32_t cid = pid[i] * 8u + (uint32_t)(lane & 7);
        const bool ok = p < pcnt && cid < (uint32_t)gl;
        pid[i] = ok ? pid[i] : 0xFFFFFFFFu;
        kr[i] = src[ok ? cid : 0u];
      }
      if (pool_pending) {                // the previous round's pool, while the gathers fly
        if (write) write_pool(pcnt, par);
        pool_pending = false;
      }
      // all gathers in flight before the first use (left to itself the
      // compiler sinks each load to its use and serialises their latencies)
      __builtin_amdgcn_s_waitcnt(0);
      // children below the floor stay: the round's key bounds leave them out
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t k = is_score ? f32_key(__uint_as_float(kr[i])) : kr[i];
        kr[i] = pid[i] != 0xFFFFFFFFu ? k : 0u;
      }
    }
    const int want = (lvl == 0 && mode == 1) ? k2 : kk;
    const bool fr = first;
    const RoundOut ro = select_round<NT, PER>(
        kr, !first, floor_key > 0u ? floor_key : 1u, top_key, want, sh, sh.lists[cur ^ 1],
        [&](int i) __attribute__((always_inline)) {
          return fr ? (uint32_t)(cbase + 64 * i) : pid[i] * 8u + (uint32_t)(lane & 7);
        });
    const int kept = ro.kept;
    cur ^= 1;
    first = false;
    pcnt = kept;
    top_key = ro.mx;
    const uint32_t* sel = sh.lists[cur];
    const bool map_cols = lvl == stop && mode == 0 && col_ids;

    if (lvl == stop && mode == 0) {
      if (write) {
        for (int i = tid; i < kk; i += NT) {
          int32_t o = -1;
          if (i < kept) o = map_cols ? col_ids[(int64_t)q * ld + sel[i]] : (int32_t)sel[i];
          orow[i] = o;
        }
      }
      return SelResult{kept, false, sel};
    }
    if (lvl == 1 && mode == 1) {           // the pool: positions of the kept blocks
      if (k2 <= 0) {
        if (write) write_pool(kept, sel);
        return SelResult{kept, false, sel};
      }
      pool_pending = true;                 // written while the next round loads
    }
    if (lvl == 0 && mode == 1) {           // the Full layer's own top-k, from inside its pool
      if (write) {
        for (int i = tid; i < k2; i += NT)
          out2[(int64_t)q * k2 + i] = i < kept ? (int32_t)sel[i] : -1;
      }
      return SelResult{kept, false, sel};
    }
    --lvl;
    const int want_next = (lvl == 0 && mode == 1) ? k2 : kk;
    floor_key = kept >= want_next ? (ro.all ? ro.mn : ro.lo) : 0u;
  }
}


// Host side (select.hip): the pyramid levels a selection over n_cols
// columns needs (mode 0 top-k, mode 1 block pool) and the launch of the
// maxima kernel that fills them into ws.
LevelDesc select_levels(int Q, int64_t n_cols, int mode);
hipError_t launch_maxima(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                         int64_t n_cols, const LevelDesc& d, uint32_t* ws, hipStream_t stream);

}  // namespace csa2
