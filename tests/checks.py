"""Parity checks of the HIP path against the fp64 oracle.

Each check takes the GPU's outputs (copied to the host) and the inputs both
sides saw, recomputes the step with the oracle and asserts the bar:
  * m = 1 main-KV codes and scales: bit-exact.
  * indexer-K codes (fp32 projection on the GPU) and m = 2 main-KV codes
    (fp32 pooling on the GPU): equal, except where the oracle's value lies
    within the GPU arithmetic's error bound of a rounding threshold; there
    the GPU's code must be one of the two codes the threshold separates.
  * scores: |s - r| <= 1e-3 * max(|r|, 1e-3 * max_j |r_j|).
  * top-k and pool computed from the GPU's own fp32 scores: bit-exact
    against the oracle's selection on the same fp32 values; against the
    oracle's fp64 scores, the sets may differ only in entries whose fp64
    score is within 1e-5 relative of the k-th score.
  * attention: max|o - o_ref| / max|o_ref| <= 2e-3; per head
    |lse - lse_ref| <= 1e-4 absolute on the workloads' inputs; rows spread
    over many binades (stress tests, logits far above the workloads' O(1))
    are judged at 1e-4 of the head's largest |logit|, as the output is
    judged relative to its own magnitude.
  * FP8 SWA rows: the fp32 row scale bit-exact; codes equal except where the
    oracle's exact quotient lies within 2^-22 relative of an E4M3 rounding
    midpoint, where the GPU's code must be one of the two it separates.
  * top-k and pool against the fp64 scores of every visible entry: the sets
    differ only in near-ties (1e-5 relative of the k-th score or of the
    n_blocks-th block maximum).
Stages hand off the GPU's own results (cache bytes, pool, indices) to the
oracle's next stage, since a near-tie swap changes which rows are read.
"""
import numpy as np
import torch

from oracle import csa2_ref as R
from oracle import formats as F

SCORE_RTOL = 1e-3
TIE_RTOL = 1e-5
ATT_TOL = 2e-3
LSE_ATOL = 1e-4

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_E4M3_POS = F.e4m3fn_value(np.arange(0x7F))
E4M3_MIDS = (_E4M3_POS[1:] + _E4M3_POS[:-1]) / 2


def host(t):
    return t.detach().cpu().numpy()


def bf16_to_f64(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


# ----------------------------------------------------------------- codes
def _near(vals, mids, tol):
    """|vals| within tol of any midpoint (elementwise)."""
    a = np.abs(vals)[..., None]
    return (np.abs(a - mids) <= tol[..., None]).any(-1)


def check_codes_with_margin(ref_vals, delta, gpu_codes, gpu_scales, ref_codes, ref_scales,
                            group, scale_value, scale_mids, elem_div_scale=True):
    """Compare GPU nibble codes / scale bytes with the oracle's under the
    margin rule.  ref_vals [n, C] are the oracle's pre-quantisation values,
    delta [n, C] the GPU error bound; scale_value maps scale bytes to
    values; scale_mids are the rounding thresholds of the scale (None for
    E8M0: thresholds are powers of two)."""
    n, C = ref_vals.shape
    G = C // group
    rv = ref_vals.reshape(n, G, group)
    dl = delta.reshape(n, G, group)
    amax = np.abs(rv).max(-1)
    dmax = dl.max(-1)
    bad_scale = gpu_scales != ref_scales
    if bad_scale.any():
        if scale_mids is None:                       # E8M0: floor(log2 amax) boundary
            p = np.exp2(np.round(np.log2(np.maximum(amax, 1e-300))))
            ok = np.abs(amax - p) <= dmax
        else:                                        # E4M3: amax / 6 near a midpoint
            ok = _near(amax / 6.0, scale_mids, dmax / 6.0)
        assert ok[bad_scale].all(), f"{int((bad_scale & ~ok).sum())} scale bytes differ beyond the margin"
    # element codes, judged against the scale the GPU chose
    s = scale_value(gpu_scales)[..., None]
    gc = F.unpack_nibbles(gpu_codes).reshape(n, G, group)
    rc = F.unpack_nibbles(ref_codes).reshape(n, G, group)
    safe = np.where(s > 0, s, 1.0)
    want = np.where(s > 0, F.e2m1_encode(rv / safe), 0)
    # canonical zero: +0 and -0 are the same value
    mag = lambda c: np.where((c & 7) == 0, 0, c)
    diff = mag(gc) != mag(want)
    if diff.any():
        near = _near(rv / safe, E2M1_MIDS, dl / safe)
        adj = np.abs(F.e2m1_value(gc) - F.e2m1_value(want)) <= 2.0 + 1e-12
        ok = near & adj
        assert ok[diff].all(), f"{int((diff & ~ok).sum())} codes differ beyond the margin"
    return int(diff.sum()), int(bad_scale.sum())


def check_main_kv(x_ref, m, gpu_kv_codes, gpu_kv_scales, h_abs_max):
    """a1 + a2: oracle pooled x (fp64) quantised vs the GPU's bytes."""
    rc, rs = R.quant_main_kv(x_ref)
    if m == 1:
        assert np.array_equal(gpu_kv_scales, rs), "main-KV scales differ (m=1 must be exact)"
        g = F.unpack_nibbles(gpu_kv_codes)
        r = F.unpack_nibbles(rc)
        assert np.array_equal(g, r), f"main-KV codes differ at {int((g != r).sum())} channels (m=1)"
        return 0, 0
    # fp32 pooling: a few ulp of the largest input of the group of m rows
    delta = np.asarray(h_abs_max, np.float64) * 2.0 ** -18
    return check_codes_with_margin(x_ref, delta, gpu_kv_codes, gpu_kv_scales, rc, rs, 16,
                                   F.e4m3fn_value, E4M3_MIDS)


def check_indexer_k(gpu_kv_codes, gpu_kv_scales, w_ik, gpu_ik_codes, gpu_ik_scales):
    """a3, stage-wise: the oracle projects the GPU's stored main KV."""
    xhat = R.dequant_main_kv(gpu_kv_codes, gpu_kv_scales)
    k = R.project_indexer_k(xhat, w_ik)
    rc, rs = R.quant_mxfp4(k)
    # fp32 accumulation of 512 exact products: bound n * 2^-24 * sum|terms|, doubled
    delta = (np.abs(xhat) @ np.abs(w_ik).T) * (2 * 512 * 2.0 ** -24)
    return check_codes_with_margin(k, delta, gpu_ik_codes, gpu_ik_scales, rc, rs, 32,
                                   F.e8m0_value, None)


# ---------------------------------------------------------------- scores
def check_scores(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    floor = max(1e-3 * np.abs(ref).max(), np.finfo(np.float64).tiny)
    tol = SCORE_RTOL * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu - ref)
    assert np.all(err <= tol), f"scores: max rel err {float((err / np.maximum(np.abs(ref), floor)).max()):.3e}"
    return float((err / np.maximum(np.abs(ref), floor)).max())


def check_topk_exact(gpu_idx, scores_f32, k, ids=None):
    """The GPU selection equals the oracle's selection on the same fp32 scores."""
    want = R.topk(np.asarray(scores_f32, np.float64), k, ids)
    got = np.sort(gpu_idx[gpu_idx >= 0])
    assert got.size == min(k, len(scores_f32)), f"count {got.size} != {min(k, len(scores_f32))}"
    assert np.array_equal(got, want), f"top-k differs in {np.setxor1d(got, want).size} ids"
    assert np.all(gpu_idx[got.size:] == -1), "padding after the selected ids must be -1"
    assert np.all(np.diff(gpu_idx[:got.size]) > 0), "selected ids must be ascending"


def check_topk_tolerance(gpu_idx, ref_scores, k, ids=None):
    """Against fp64 scores: only near-ties (within 1e-5 of the k-th) may swap."""
    ref_scores = np.asarray(ref_scores, np.float64)
    ids = np.arange(ref_scores.size) if ids is None else np.asarray(ids)
    want = R.topk(ref_scores, k, ids)
    got = np.sort(gpu_idx[gpu_idx >= 0])
    assert got.size == want.size
    sd = np.setxor1d(got, want)
    if sd.size:
        kth = R.kth_score(ref_scores, k)
        pos = {int(e): i for i, e in enumerate(ids)}
        s = np.array([ref_scores[pos[int(e)]] for e in sd])
        assert np.all(np.abs(s - kth) <= TIE_RTOL * abs(kth)), "top-k swap beyond the tie tolerance"
    return int(sd.size)


def check_pool_exact(gpu_pool, gpu_len, scores_f32, block, n_blocks):
    want = R.block_pool(np.asarray(scores_f32, np.float64), block, n_blocks)
    assert int(gpu_len) == want.size, f"pool_len {int(gpu_len)} != {want.size}"
    assert np.array_equal(gpu_pool[:want.size], want), "pool differs"
    assert np.all(gpu_pool[want.size:] == -1)


# ------------------------------------------------------------- attention
def _lse_tol(q, rows, lse_scale):
    """Per-head LSE bar: 1e-4 absolute, or with lse_scale 1e-4 of the head's
    largest |logit| (never below 1e-4)."""
    if not lse_scale:
        return LSE_ATOL
    lmax = np.abs(np.asarray(q, np.float64) @ np.asarray(rows, np.float64).T).max(axis=1)
    return LSE_ATOL * np.maximum(1.0, lmax)


def check_attention(o_gpu, lse_gpu, q, rows, lse_scale=False):
    o_ref, lse_ref = R.attend(q, rows)
    # normalised by the output's magnitude; an all-zero output (every
    # attended row zero) must come out exactly zero
    scale = np.abs(o_ref).max()
    if scale == 0:
        assert np.all(o_gpu == 0), "non-zero attention output over zero rows"
        scale = 1.0
    err = np.abs(o_gpu - o_ref).max() / scale
    assert err <= ATT_TOL, f"attention err {err:.3e}"
    ltol = _lse_tol(q, rows, lse_scale)
    lerr = np.abs(lse_gpu - lse_ref)
    assert np.all(lerr <= ltol), f"lse err {float(lerr.max()):.3e} (tol {float(np.min(ltol)):.3e})"
    return float(err), float(lerr.max())


def check_attention_bf16(o_gpu_bf16, lse_gpu, o_ref, lse_ref, q, rows, lse_scale=False):
    """bf16 output of the fused RoPE kernel against the oracle's output
    before its cast: the fp32 error bound of check_attention, plus the bf16
    rounding of the fp32 value (8 significant bits: at most 2^-8 of its
    magnitude)."""
    o = np.asarray(o_gpu_bf16, np.float64)
    scale = np.abs(o_ref).max()
    if scale == 0:
        assert np.all(o == 0), "non-zero attention output over zero rows"
        scale = 1.0
    tol = ATT_TOL * scale * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(o_ref)
    err = np.abs(o - o_ref)
    assert np.all(err <= tol), f"bf16 attention err {float((err / scale).max()):.3e}"
    ltol = _lse_tol(q, rows, lse_scale)
    lerr = np.abs(lse_gpu - lse_ref)
    assert np.all(lerr <= ltol), f"lse err {float(lerr.max()):.3e}"
    return float((err / scale).max())


def swa_rows(swa_codes, swa_scale, start, length):
    """The SWA window as the attention reads it: a ring of T_swa slots."""
    T = len(swa_scale)
    length = min(length, T) if 0 <= start < T else 0
    if length <= 0:
        return None, None
    return R.swa_window(swa_codes, swa_scale, start, length)


def check_swa_rows(gpu_codes, gpu_sigma, x):
    """FP8 SWA rows written on the GPU against R.quant_swa_row of the same
    latents x [r, 512]: the fp32 scale bit-exact; a code may differ only
    where the exact quotient x / sigma lies within 2^-22 relative of an
    E4M3 rounding midpoint (one fp32 division rounds it by at most 2^-24),
    and then it must be one of the two neighbouring codes.  Returns the
    number of such codes."""
    rc, rs = R.quant_swa_row(x)
    gpu_codes = np.asarray(gpu_codes)
    gpu_sigma = np.asarray(gpu_sigma, np.float32)
    assert np.array_equal(gpu_sigma, rs), "SWA row scales differ"
    s64 = rs.astype(np.float64)
    v = np.asarray(x, np.float64) / np.where(s64 > 0, s64, 1.0)[..., None]
    gv = F.e4m3fn_value(gpu_codes)
    rv = F.e4m3fn_value(rc)
    diff = gv != rv                        # -0 and +0 decode equal
    if diff.any():
        near = _near(v, E4M3_MIDS, np.abs(v) * 2.0 ** -22)
        lo = np.minimum(np.abs(gv), np.abs(rv))
        hi = np.maximum(np.abs(gv), np.abs(rv))
        # adjacent: no representable value strictly between them
        adj = ~((_E4M3_POS[None, :] > lo.reshape(-1, 1)) & (_E4M3_POS[None, :] < hi.reshape(-1, 1))).any(1)
        adj = adj.reshape(lo.shape) & (np.sign(gv) * np.sign(rv) >= 0)
        ok = near & adj
        assert ok[diff].all(), f"{int((diff & ~ok).sum())} SWA codes differ beyond the margin"
    return int(diff.sum())


def full_index_scores(q_idx, w, ik_codes, ik_scales, n, chunk=1 << 16):
    """The oracle's fp64 scores of one query against entries 0..n-1, the
    entries dequantised and scored a chunk at a time (memory only: each
    score depends on its own entry)."""
    out = np.empty(n)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        out[i:j] = R.index_scores(q_idx, w, R.dequant_mxfp4(ik_codes[i:j], ik_scales[i:j]))
    return out


def check_pool_tolerance(gpu_pool, gpu_len, ref_scores, block, n_blocks):
    """The GPU's pool against the oracle's pool on fp64 scores: the same
    length, and the kept block sets may differ only in blocks whose fp64
    maximum is within 1e-5 relative of the n_blocks-th best block maximum.
    Returns the number of swapped blocks."""
    want = R.block_pool(np.asarray(ref_scores, np.float64), block, n_blocks)
    got = np.asarray(gpu_pool)[:int(gpu_len)]
    assert int(gpu_len) == want.size, f"pool_len {int(gpu_len)} != {want.size}"
    assert np.all(np.asarray(gpu_pool)[int(gpu_len):] == -1)
    assert np.all(np.diff(got) > 0), "pool must be ascending"
    gb, wb = np.unique(got // block), np.unique(want // block)
    # every kept block contributes all of its visible positions
    n = len(ref_scores)
    full = lambda b: np.concatenate([np.arange(x * block, min(n, x * block + block)) for x in b]) if len(b) else np.zeros(0, np.int64)
    assert np.array_equal(got, full(gb)), "pool does not cover whole blocks"
    sd = np.setxor1d(gb, wb)
    if sd.size:
        bmax = R.block_max(ref_scores, block)
        kth = R.kth_score(bmax, n_blocks)
        assert np.all(np.abs(bmax[sd] - kth) <= TIE_RTOL * abs(kth)), "pool swap beyond the tie tolerance"
    return int(sd.size)


# ------------------------------------------------------------- one step
def check_step(step, q_sample=None):
    """Check every layer of an executed Step (run with keep=True) against the
    oracle, stage by stage: every Full-layer score against the oracle's fp64
    score of that entry, the Full layer's top-k (and pool) both exactly
    against a selection over the GPU's own fp32 scores and against the fp64
    ranking within the tie tolerance, every Reindex score and selection,
    and every attention output.  q_sample limits the queries checked."""
    wl = step.wl
    cache = {k: v for k, v in step.cache.arrays().items()}
    q_seq = host(step.q_seq)
    n_vis = host(step.n_vis)
    swa_start = host(step.swa_start)
    swa_len = host(step.swa_len)
    Q = wl.Q
    qs = np.arange(Q) if q_sample is None else np.asarray(q_sample)
    seqs = sorted(set(int(q_seq[q]) for q in qs))
    # cache of the sequences involved, on the host
    kv_c = {b: host(cache["kv_codes"][b]) for b in seqs}
    kv_s = {b: host(cache["kv_scales"][b]) for b in seqs}
    ik_c = {b: host(cache["ik_codes"][b]) for b in seqs}
    ik_s = {b: host(cache["ik_scales"][b]) for b in seqs}
    report = {"topk_swaps": 0, "pool_swaps": 0}
    for li, mode in enumerate(wl.layers):
        L = step.layers[li]
        q_idx = bf16_to_f64(L["q_idx"])
        w = host(L["w"]).astype(np.float64)
        q_att = bf16_to_f64(L["q_attn"])
        sw_c = host(L["swa_codes"])
        sw_s = host(L["swa_scale"]).astype(np.float64)
        idx = host(step.idx_per_layer[li])
        sc_gpu = host(step.scores_per_layer[li]) if step.scores_per_layer[li] is not None else None
        if mode == "reindex":
            pool = host(step.pool)
            plen = host(step.pool_len)
        for q in qs:
            b = int(q_seq[q])
            nv = int(n_vis[q])
            if mode == "full":
                s_g = sc_gpu[q, :nv]
                ref = full_index_scores(q_idx[q], w[q], ik_c[b], ik_s[b], nv)
                check_scores(s_g, ref)
                check_topk_exact(idx[q], s_g, wl.k)
                report["topk_swaps"] += check_topk_tolerance(idx[q], ref, wl.k)
                if wl.hierarchical:
                    check_pool_exact(host(step.pool[q]), host(step.pool_len[q]), s_g, wl.block,
                                     wl.n_blocks)
                    report["pool_swaps"] += check_pool_tolerance(
                        host(step.pool[q]), host(step.pool_len[q]), ref, wl.block, wl.n_blocks)
            elif mode == "reindex":
                pl = int(plen[q])
                ids = pool[q, :pl]
                s_g = sc_gpu[q, :pl]
                ref = R.index_scores(q_idx[q], w[q], R.dequant_mxfp4(ik_c[b][ids], ik_s[b][ids]))
                check_scores(s_g, ref)
                check_topk_exact(idx[q], s_g, wl.k, ids)
                report["topk_swaps"] += check_topk_tolerance(idx[q], ref, wl.k, ids)
            # attention over the GPU's own selection (a8 + a9)
            sc, ss = swa_rows(sw_c[b], sw_s[b], int(swa_start[q]), int(swa_len[q]))
            rows = R.gather_rows(kv_c[b], kv_s[b], idx[q], sc, ss)
            check_attention(host(step.out[li][q]), host(step.lse[li][q]), q_att[q], rows)
    return report
