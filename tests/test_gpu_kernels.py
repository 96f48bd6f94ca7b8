"""Per-operation parity of the HIP kernels against the fp64 oracle, through
the C ABI, at sizes the oracle finishes in seconds (several tiles plus a
ragged tail) and on the edge cases (empty, ragged, ties, k > n, masked rows,
empty SWA window, split and unsplit attention)."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_csa2_amd as C
from long_context_sparse_csa2_amd import synth
from oracle import csa2_ref as R
from oracle import formats as F
from tests import checks

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _latents(B, T, seed, scale_rows=True):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, T, 512, generator=g)
    if scale_rows:   # spread magnitudes over many binades to exercise every scale code
        h = h * torch.exp(torch.empty(B, T, 1).uniform_(-9, 6, generator=g))
    z = torch.randn(B, T, 512, generator=g) * 2
    return h.to(torch.bfloat16), z.to(torch.bfloat16)


def _build(B, T, m, seed):
    h, z = _latents(B, T, seed)
    w = (torch.randn(128, 512, generator=torch.Generator().manual_seed(seed + 7)) / math.sqrt(512)).to(torch.bfloat16)
    cache = C.Cache(B, T // m, DEV)
    C.csa2_compress_quant(h.to(DEV), z.to(DEV) if m > 1 else None, m, w.to(DEV), cache)
    torch.cuda.synchronize()
    return h, z, w, cache


def test_selftest():
    assert C.csa2_selftest(DEV) == [0] * 9


@pytest.mark.parametrize("m,T", [(1, 1000), (2, 2000), (4, 4 * 77)])
def test_compress_quant(m, T):
    B = 2
    h, z, w, cache = _build(B, T, m, seed=10 + m)
    w64 = checks.bf16_to_f64(w)
    for b in range(B):
        h64 = checks.bf16_to_f64(h[b])
        z64 = checks.bf16_to_f64(z[b])
        x = R.compress(h64, z64, m)
        hmax = np.abs(h64).reshape(-1, m, 512).max(1)
        kv_c, kv_s = checks.host(cache.kv_codes[b]), checks.host(cache.kv_scales[b])
        checks.check_main_kv(x, m, kv_c, kv_s, hmax)
        checks.check_indexer_k(kv_c, kv_s, w64, checks.host(cache.ik_codes[b]),
                               checks.host(cache.ik_scales[b]))


def test_compress_offset_and_tail():
    # e0 offset and an entry count that is not a multiple of the 32-entry tile
    h, z = _latents(1, 45, 3)
    w = (torch.randn(128, 512, generator=torch.Generator().manual_seed(5)) / 22.6).to(torch.bfloat16)
    cache = C.Cache(1, 100, DEV)
    cache.kv_codes.fill_(0xAB)
    C.csa2_compress_quant(h.to(DEV), None, 1, w.to(DEV), cache, e0=50)
    torch.cuda.synchronize()
    kv = checks.host(cache.kv_codes[0])
    assert np.all(kv[:50] == 0xAB) and np.all(kv[95:] == 0xAB)
    rc, rs = R.quant_main_kv(checks.bf16_to_f64(h[0]))
    assert np.array_equal(kv[50:95], rc)
    assert np.array_equal(checks.host(cache.kv_scales[0])[50:95], rs)


def _scores_inputs(Q, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(Q, 32, 128, generator=g).to(torch.bfloat16)
    w = torch.rand(Q, 32, generator=g)
    return q, w


def test_index_score_full_and_pool():
    B, T = 2, 3000
    _, _, _, cache = _build(B, T, 1, seed=21)
    Q = 3
    q, w = _scores_inputs(Q, 22)
    q_seq = torch.tensor([0, 1, 1], dtype=torch.int32)
    n_vis = torch.tensor([3000, 2999, 1], dtype=torch.int64)
    scores = torch.full((Q, 3008), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq.to(DEV), n_vis.to(DEV), None, 3000, cache, scores)
    torch.cuda.synchronize()
    s = checks.host(scores)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    for i in range(Q):
        b, nv = int(q_seq[i]), int(n_vis[i])
        khat = R.dequant_mxfp4(checks.host(cache.ik_codes[b]), checks.host(cache.ik_scales[b]))
        checks.check_scores(s[i, :nv], R.index_scores(q64[i], w64[i], khat[:nv]))
        assert np.all(s[i, nv:] == -7.0)          # unscored columns untouched
    # candidate mode (Reindex): arbitrary ascending entry ids
    rng = np.random.default_rng(0)
    cand = np.full((Q, 700), -1, dtype=np.int32)
    lens = [700, 333, 0]
    for i in range(Q):
        cand[i, :lens[i]] = np.sort(rng.choice(2999, lens[i], replace=False))
    ps = torch.full((Q, 700), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq.to(DEV), torch.tensor(lens, dtype=torch.int64).to(DEV),
                       torch.from_numpy(cand).to(DEV), 700, cache, ps)
    torch.cuda.synchronize()
    p = checks.host(ps)
    for i in range(Q):
        b = int(q_seq[i])
        ids = cand[i, :lens[i]]
        khat = R.dequant_mxfp4(checks.host(cache.ik_codes[b])[ids], checks.host(cache.ik_scales[b])[ids])
        checks.check_scores(p[i, :lens[i]], R.index_scores(q64[i], w64[i], khat))
        assert np.all(p[i, lens[i]:] == -7.0)


def _random_indexer_cache(B, cap, seed):
    """A cache whose indexer K holds random E2M1 codes and E8M0 scales in
    2^-7 .. 2^7 (the scan reads nothing else)."""
    g = torch.Generator().manual_seed(seed)
    cache = C.Cache(B, cap, DEV)
    cache.ik_codes.copy_(torch.randint(0, 256, (B, cap, 64), generator=g, dtype=torch.uint8))
    cache.ik_scales.copy_(torch.randint(120, 135, (B, cap, 4), generator=g, dtype=torch.uint8))
    return cache


@pytest.mark.parametrize("fp4q", [False, True])
def test_index_score_long_ragged(fp4q):
    # 600,000 columns for 3 queries: 8 tiles per wave and workgroups that
    # interleave 128-column slices over the whole row, so a query whose
    # visible count ends mid-row has waves with tiles on both sides of it
    # (and one query sees nothing)
    B, cap, Q, N = 2, 600_000, 3, 600_000
    cache = _random_indexer_cache(B, cap, 91)
    q, w = _scores_inputs(Q, 92)
    q_seq = torch.tensor([0, 1, 0], dtype=torch.int32)
    n_vis = [N - 13, 250_001, 0]
    scores = torch.full((Q, N), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq.to(DEV), torch.tensor(n_vis, dtype=torch.int64).to(DEV),
                       None, N, cache, scores, fp4q=fp4q)
    torch.cuda.synchronize()
    s = checks.host(scores)
    codes, scl = checks.host(cache.ik_codes), checks.host(cache.ik_scales)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    rng = np.random.default_rng(93)
    for i in range(Q):
        nv, b = n_vis[i], int(q_seq[i])
        assert np.all(s[i, nv:] == -7.0)                 # columns past n_vis untouched
        if nv == 0:
            continue
        cols = np.unique(np.concatenate([rng.choice(nv, 3000, replace=False), np.arange(min(nv, 64)),
                                         np.arange(max(0, nv - 64), nv)]))
        khat = R.dequant_mxfp4(codes[b][cols], scl[b][cols])
        ref = (_oracle_scores_fp4q(q64[i], w64[i], khat) if fp4q
               else R.index_scores(q64[i], w64[i], khat))
        checks.check_scores(s[i, cols], ref)


def _device_indexer_cache(cap, seed):
    """One sequence of random MXFP4 indexer keys generated on the device (the
    scan reads only the indexer arrays; the main-KV arrays are one entry)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    cache = C.Cache.__new__(C.Cache)
    cache.B, cache.cap = 1, cap
    cache.kv_codes = torch.zeros(1, 1, 256, dtype=torch.uint8, device=DEV)
    cache.kv_scales = torch.zeros(1, 1, 32, dtype=torch.uint8, device=DEV)
    cache.ik_codes = torch.randint(0, 256, (1, cap, 64), generator=g, dtype=torch.uint8, device=DEV)
    cache.ik_scales = torch.randint(120, 135, (1, cap, 4), generator=g, dtype=torch.uint8, device=DEV)
    return cache


@pytest.mark.parametrize("fp4q", [False, True])
@pytest.mark.parametrize("N", [(1 << 24) + 4100, (1 << 25) + 4100])
def test_index_score_longest_rows(N, fp4q):
    # rows past the length up to which workgroups interleave their tiles
    # (2^24 columns) and past 2^25 columns, where a workgroup addresses its
    # keys from its own first column: sampled columns at the row's start and
    # end, around those lengths and the workgroup chunk edges, against the
    # oracle; a query that ends mid-row leaves the rest of its row untouched
    Q = 2
    print(f"[longest rows] N={N} fp4q={fp4q}", flush=True)
    cache = _device_indexer_cache(N, 95)
    q, w = _scores_inputs(Q, 96)
    n_vis = [N, N - 4133]
    scores = torch.full((Q, N), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.zeros(Q, dtype=torch.int32, device=DEV),
                       torch.tensor(n_vis, dtype=torch.int64).to(DEV), None, N, cache, scores,
                       fp4q=fp4q)
    torch.cuda.synchronize()
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    rng = np.random.default_rng(97)
    for i in range(Q):
        nv = n_vis[i]
        edges = [0, 4096, (1 << 24) - 64, 1 << 24, (1 << 25) - 64, 1 << 25, nv - 4096 - 64, nv - 128]
        cols = np.unique(np.concatenate([rng.choice(nv, 2000, replace=False)] +
                                        [np.arange(e, e + 128) for e in edges]))
        cols = cols[(cols >= 0) & (cols < nv)]
        idx = torch.from_numpy(cols).to(DEV)
        got = checks.host(scores[i].index_select(0, idx))
        khat = R.dequant_mxfp4(checks.host(cache.ik_codes[0].index_select(0, idx)),
                               checks.host(cache.ik_scales[0].index_select(0, idx)))
        ref = (_oracle_scores_fp4q(q64[i], w64[i], khat) if fp4q
               else R.index_scores(q64[i], w64[i], khat))
        checks.check_scores(got, ref)
        assert bool((scores[i, nv:] == -7.0).all())


def test_select_at_max_columns():
    # CSA2_MAX_COLS columns (the largest selection row), full and ragged:
    # top-512, top-2048 and the 2048-block pool with its top-512
    n = C.CSA2_MAX_COLS
    Q = 2
    s = _rand_scores(Q, n, seed=98)
    nv = [n, n - 1001]
    for k, rows in ((512, (0, 1)), (2048, (1,))):     # (the oracle's ranking of 2^24 takes seconds)
        out = _topk(s, nv, k)
        for i in rows:
            checks.check_topk_exact(out[i], s[i, :nv[i]], k)
    ws = C.workspace(C.CSA2_OP_POOL, Q, n, 2048, DEV)
    pool = torch.empty(Q, 16384, dtype=torch.int32, device=DEV)
    plen = torch.empty(Q, dtype=torch.int64, device=DEV)
    topk = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    C.csa2_block_pool(torch.from_numpy(s).to(DEV), torch.tensor(nv, dtype=torch.int64).to(DEV), n,
                      2048, pool, plen, ws, topk=topk)
    torch.cuda.synchronize()
    for i in range(Q):
        checks.check_pool_exact(checks.host(pool[i]), checks.host(plen[i]), s[i, :nv[i]], 8, 2048)
        checks.check_topk_exact(checks.host(topk[i]), s[i, :nv[i]], 512)


def test_index_score_candidates_multi_tile():
    # 64 queries over 4,096 candidate columns: two tiles per wave, so
    # workgroups and tiles past a query's candidate count score entry 0 and
    # drop their stores; the padding ids past the count are -1
    B, cap, Q, N = 2, 5000, 64, 4096
    cache = _random_indexer_cache(B, cap, 94)
    q, w = _scores_inputs(Q, 95)
    rng = np.random.default_rng(96)
    q_seq = (np.arange(Q) % B).astype(np.int32)
    lens = rng.integers(0, N + 1, Q)
    lens[:4] = [N, 0, 1, 33]
    cand = np.full((Q, N), -1, dtype=np.int32)
    for i in range(Q):
        cand[i, :lens[i]] = rng.choice(cap, lens[i], replace=False)
    ps = torch.full((Q, N), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.from_numpy(q_seq).to(DEV),
                       torch.from_numpy(lens.astype(np.int64)).to(DEV), torch.from_numpy(cand).to(DEV),
                       N, cache, ps)
    torch.cuda.synchronize()
    p = checks.host(ps)
    codes, scl = checks.host(cache.ik_codes), checks.host(cache.ik_scales)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    for i in range(Q):
        n, b = int(lens[i]), int(q_seq[i])
        assert np.all(p[i, n:] == -7.0)
        if n:
            ids = cand[i, :n]
            checks.check_scores(p[i, :n], R.index_scores(q64[i], w64[i], R.dequant_mxfp4(codes[b][ids], scl[b][ids])))


def _fp4q_special_queries(Q, seed):
    """Indexer queries that exercise the MXFP4 query quantiser: per-block
    magnitudes spread over 2^-30 .. 2^20, exact E2M1 ties (0.25, 0.75, 1.25,
    1.75, 2.5, 3.5, 5 times the block scale), all-zero blocks, negative
    zeros, blocks whose scale clamps at 2^-127, and saturation (|q| / X in
    (6, 8))."""
    q, w = _scores_inputs(Q, seed)
    g = torch.Generator().manual_seed(seed + 1)
    ex = torch.randint(-30, 21, (Q, 32, 4, 1), generator=g).float()
    q = (q.float().reshape(Q, 32, 4, 32) * torch.exp2(ex)).reshape(Q, 32, 128)
    ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -2.5, -0.25, 6.0])
    q[0, 1, 32:42] = ties * 2.0 ** -7            # amax 6 X with X = 2^-7
    q[0, 2, 64:96] = 0.0                          # all-zero block
    q[0, 3, 0:32] = -0.0                          # negative zeros only
    q[0, 4, 96:128] = 0.0
    q[0, 4, 96] = 2.0 ** -130                     # scale clamps at 2^-127: 2^-130 / X = 1/8
    q[0, 4, 97] = -2.0 ** -126                    # 2 X: exact
    q[0, 5, 0:32] = 0.0
    q[0, 5, 0] = 7.5                              # X = 1: saturates to 6
    q[0, 5, 1] = -7.0
    q[0, 5, 2] = 1.0
    return q.to(torch.bfloat16), w


def _oracle_scores_fp4q(q64, w64, khat):
    return R.index_scores_fp4q(q64, w64, khat)


@pytest.mark.parametrize("special", [False, True])
def test_index_score_fp4q(special):
    """MXFP4-query scoring (full scan and candidate pool) against the oracle's
    quantised query."""
    B, T, Q = 2, 3000, 5
    _, _, _, cache = _build(B, T, 1, seed=31)
    q, w = _fp4q_special_queries(Q, 32) if special else _scores_inputs(Q, 32)
    q_seq = torch.tensor([0, 1, 1, 0, 1], dtype=torch.int32)
    n_vis = torch.tensor([3000, 2999, 1, 257, 2049], dtype=torch.int64)
    scores = torch.full((Q, 3008), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq.to(DEV), n_vis.to(DEV), None, 3000, cache,
                       scores, fp4q=True)
    torch.cuda.synchronize()
    s = checks.host(scores)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    khat = [R.dequant_mxfp4(checks.host(cache.ik_codes[b]), checks.host(cache.ik_scales[b])) for b in range(B)]
    for i in range(Q):
        b, nv = int(q_seq[i]), int(n_vis[i])
        checks.check_scores(s[i, :nv], _oracle_scores_fp4q(q64[i], w64[i], khat[b][:nv]))
        assert np.all(s[i, nv:] == -7.0)
    # candidate mode
    rng = np.random.default_rng(3)
    P = 900
    lens = [900, 333, 0, 1, 64]
    cand = np.full((Q, P), -1, dtype=np.int32)
    for i in range(Q):
        cand[i, :lens[i]] = np.sort(rng.choice(2999, lens[i], replace=False))
    ps = torch.full((Q, P), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq.to(DEV), torch.tensor(lens, dtype=torch.int64).to(DEV),
                       torch.from_numpy(cand).to(DEV), P, cache, ps, fp4q=True)
    torch.cuda.synchronize()
    p = checks.host(ps)
    for i in range(Q):
        b = int(q_seq[i])
        ids = cand[i, :lens[i]]
        if lens[i]:
            checks.check_scores(p[i, :lens[i]], _oracle_scores_fp4q(q64[i], w64[i], khat[b][ids]))
        assert np.all(p[i, lens[i]:] == -7.0)


def test_index_score_fp4q_many_queries():
    """300 queries over mixed sequences and ragged visible counts, and the
    top-512 of the resulting scores equal to the oracle's selection."""
    B, T, Q = 3, 1000, 300
    _, _, _, cache = _build(B, T, 1, seed=33)
    q, w = _scores_inputs(Q, 34)
    rng = np.random.default_rng(7)
    q_seq = rng.integers(0, B, Q).astype(np.int32)
    n_vis = (np.arange(Q) * 13 % (T + 1)).astype(np.int64)
    n_vis[:10] = T
    scores = torch.full((Q, 1008), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.from_numpy(q_seq).to(DEV),
                       torch.from_numpy(n_vis).to(DEV), None, T, cache, scores, fp4q=True)
    torch.cuda.synchronize()
    s = checks.host(scores)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    khat = [R.dequant_mxfp4(checks.host(cache.ik_codes[b]), checks.host(cache.ik_scales[b])) for b in range(B)]
    for i in range(Q):
        nv = int(n_vis[i])
        if nv:
            checks.check_scores(s[i, :nv], _oracle_scores_fp4q(q64[i], w64[i], khat[q_seq[i]][:nv]))
        assert np.all(s[i, nv:] == -7.0)
    # the fp4-query scores feed the same selection
    o = _topk(np.ascontiguousarray(s[:10]), n_vis[:10], 512)
    for i in range(10):
        checks.check_topk_exact(o[i], s[i, :T], 512)


def test_index_score_many_queries():
    """300 queries: a run sharing one sequence, then mixed sequences, ragged
    and zero visible counts, a column count that is not a multiple of the
    scan's tile."""
    B, T, Q = 3, 1000, 300
    _, _, _, cache = _build(B, T, 1, seed=23)
    q, w = _scores_inputs(Q, 24)
    rng = np.random.default_rng(5)
    q_seq = np.zeros(Q, np.int32)
    q_seq[160:] = rng.integers(0, B, Q - 160)          # mixed sequences from block 20 on
    n_vis = (np.arange(Q) * 7 % (T + 1)).astype(np.int64)
    n_vis[:40] = T
    n_vis[41] = 0
    scores = torch.full((Q, 1008), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.from_numpy(q_seq).to(DEV),
                       torch.from_numpy(n_vis).to(DEV), None, T, cache, scores)
    torch.cuda.synchronize()
    s = checks.host(scores)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    khat = [R.dequant_mxfp4(checks.host(cache.ik_codes[b]), checks.host(cache.ik_scales[b])) for b in range(B)]
    for i in range(Q):
        nv = int(n_vis[i])
        if nv:
            checks.check_scores(s[i, :nv], R.index_scores(q64[i], w64[i], khat[q_seq[i]][:nv]))
        assert np.all(s[i, nv:] == -7.0)
    # a query's scores do not depend on the other queries of the launch
    for lo, hi in ((0, 200), (100, 300)):
        part = torch.full((hi - lo, 1008), -7.0, device=DEV)
        C.csa2_index_score(q[lo:hi].to(DEV), w[lo:hi].to(DEV), torch.from_numpy(q_seq[lo:hi]).to(DEV),
                           torch.from_numpy(n_vis[lo:hi]).to(DEV), None, T, cache, part)
        torch.cuda.synchronize()
        assert np.array_equal(checks.host(part).view(np.uint32), s[lo:hi].view(np.uint32))


@pytest.mark.parametrize("fp4q,T", [(False, 40000), (True, 40000), (False, 3000), (True, 3000)])
def test_index_score_query_pairs(fp4q, T):
    """A 2049-query prefill launch over T entries (the scan scores two
    queries per wave, sharing each key tile's conversion or loads; 3000
    entries is one workgroup per pair, short causal rows) against the same
    queries in launches of 512 (one query per wave): the same score bits.
    Pairs across a sequence boundary, the last unpaired query, rows of
    different lengths within a pair and empty rows included; sampled rows
    against the oracle."""
    B, Q = 2, 2049
    _, _, _, cache = _build(B, T, 1, seed=31)
    q, w = _scores_inputs(Q, 32)
    q_seq = np.ones(Q, np.int32)
    q_seq[1001] = 0                                    # pair (1000, 1001) on two sequences
    q_seq[1500:1504] = 0                               # a run of pairs on the other one
    n_vis = np.minimum(np.arange(Q) * 19 + 1, T).astype(np.int64)
    n_vis[7] = 0                                       # an empty row beside a full one
    n_vis[40] = T
    n_vis[2048] = T - 3
    full = torch.full((Q, T), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.from_numpy(q_seq).to(DEV),
                       torch.from_numpy(n_vis).to(DEV), None, T, cache, full, fp4q=fp4q)
    parts = torch.full((Q, T), -7.0, device=DEV)
    for lo in range(0, Q, 512):
        hi = min(lo + 512, Q)
        C.csa2_index_score(q[lo:hi].to(DEV), w[lo:hi].to(DEV), torch.from_numpy(q_seq[lo:hi]).to(DEV),
                           torch.from_numpy(n_vis[lo:hi]).to(DEV), None, T, cache, parts[lo:hi],
                           fp4q=fp4q)
    torch.cuda.synchronize()
    assert bool(torch.equal(full.view(torch.int32), parts.view(torch.int32)))
    a = checks.host(full)
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    khat = [R.dequant_mxfp4(checks.host(cache.ik_codes[x]), checks.host(cache.ik_scales[x])) for x in range(B)]
    for i in (0, 1, 6, 7, 40, 41, 1000, 1001, 1500, 1503, 2047, 2048):
        nv = int(n_vis[i])
        k = khat[q_seq[i]][:nv]
        ref = _oracle_scores_fp4q(q64[i], w64[i], k) if fp4q else R.index_scores(q64[i], w64[i], k)
        checks.check_scores(a[i, :nv], ref)
        assert np.all(a[i, nv:] == -7.0)


@pytest.mark.parametrize("fp4q", [False, True])
def test_index_score_pairs_long_interleaved(fp4q):
    """2048 queries over 524,388 columns: the two-query scan with workgroups
    interleaving 128-column slices across the row, against the same queries
    in launches of 512 (one query per wave, also interleaved): the same
    score bits; ragged rows ending mid-slice; sampled columns against the
    oracle."""
    Q, N = 2048, (1 << 19) + 100
    print(f"[pairs interleaved] Q={Q} N={N} fp4q={fp4q}", flush=True)
    cache = _device_indexer_cache(N, 35)
    q, w = _scores_inputs(Q, 36)
    n_vis = (N - 37 * np.arange(Q)).astype(np.int64)
    n_vis[5] = 0
    q_seq = torch.zeros(Q, dtype=torch.int32, device=DEV)
    nv_d = torch.from_numpy(n_vis).to(DEV)
    full = torch.full((Q, N), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), q_seq, nv_d, None, N, cache, full, fp4q=fp4q)
    parts = torch.full((Q, N), -7.0, device=DEV)
    for lo in range(0, Q, 512):
        C.csa2_index_score(q[lo:lo + 512].to(DEV), w[lo:lo + 512].to(DEV), q_seq[lo:lo + 512],
                           nv_d[lo:lo + 512], None, N, cache, parts[lo:lo + 512], fp4q=fp4q)
    torch.cuda.synchronize()
    assert bool(torch.equal(full.view(torch.int32), parts.view(torch.int32)))
    del parts
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    rng = np.random.default_rng(37)
    for i in (0, 1, 4, 5, 1023, 2046, 2047):
        nv = int(n_vis[i])
        assert bool((full[i, nv:] == -7.0).all())
        if nv == 0:
            continue
        cols = np.unique(np.concatenate([rng.choice(nv, 1500, replace=False), np.arange(nv - 200, nv)]))
        idx = torch.from_numpy(cols).to(DEV)
        got = checks.host(full[i].index_select(0, idx))
        khat = R.dequant_mxfp4(checks.host(cache.ik_codes[0].index_select(0, idx)),
                               checks.host(cache.ik_scales[0].index_select(0, idx)))
        ref = _oracle_scores_fp4q(q64[i], w64[i], khat) if fp4q else R.index_scores(q64[i], w64[i], khat)
        checks.check_scores(got, ref)


def test_index_score_launch_composition():
    """A 1000-query causal launch over 5000 entries and the same queries in
    launches of 125 (which pick another tile count per wave and another
    workgroup layout): the same score bits, and sampled rows (around the
    tile and block edges) match the oracle."""
    B, T, Q = 2, 5000, 1000
    _, _, _, cache = _build(B, T, 1, seed=27)
    q, w = _scores_inputs(Q, 28)
    q_seq = np.ones(Q, np.int32)
    q_seq[997] = 0                                     # one query of the last block elsewhere
    n_vis = np.minimum(np.arange(Q) * 5 + 1, T).astype(np.int64)
    full = torch.full((Q, T), -7.0, device=DEV)
    C.csa2_index_score(q.to(DEV), w.to(DEV), torch.from_numpy(q_seq).to(DEV),
                       torch.from_numpy(n_vis).to(DEV), None, T, cache, full)
    parts = torch.full((Q, T), -7.0, device=DEV)
    for lo in range(0, Q, 125):
        hi = lo + 125
        C.csa2_index_score(q[lo:hi].to(DEV), w[lo:hi].to(DEV), torch.from_numpy(q_seq[lo:hi]).to(DEV),
                           torch.from_numpy(n_vis[lo:hi]).to(DEV), None, T, cache, parts[lo:hi])
    torch.cuda.synchronize()
    a, b = checks.host(full), checks.host(parts)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    q64, w64 = checks.bf16_to_f64(q), w.double().numpy()
    khat = [R.dequant_mxfp4(checks.host(cache.ik_codes[x]), checks.host(cache.ik_scales[x])) for x in range(B)]
    for i in (0, 1, 7, 8, 204, 205, 206, 511, 996, 997, 998, 999):
        nv = int(n_vis[i])
        checks.check_scores(a[i, :nv], R.index_scores(q64[i], w64[i], khat[q_seq[i]][:nv]))
        assert np.all(a[i, nv:] == -7.0)


def _rand_scores(Q, n, seed, ties=True):
    rng = np.random.default_rng(seed)
    s = (rng.standard_normal((Q, n)) ** 2).astype(np.float32)
    if ties:
        s[:, ::7] = np.float32(1.5)                    # many exact ties
        s[:, 3::11] = 0.0
        s[:, 5::13] = -0.0
    return s


def _topk(s, nv, k, col_ids=None):
    Q, ld = s.shape
    n_cols = int(max(nv)) if len(nv) else 0
    ws = C.workspace(C.CSA2_OP_TOPK, Q, n_cols, k, DEV)
    out = torch.empty(Q, k, dtype=torch.int32, device=DEV)
    C.csa2_select_topk(torch.from_numpy(s).to(DEV), torch.tensor(nv, dtype=torch.int64).to(DEV),
                       None if col_ids is None else torch.from_numpy(col_ids).to(DEV), n_cols, k,
                       out, ws)
    torch.cuda.synchronize()
    return checks.host(out)


@pytest.mark.parametrize("n,k", [(1, 1), (100, 512), (511, 512), (512, 512), (513, 512),
                                 (5000, 7), (6000, 2048), (9001, 600), (16384, 1), (16384, 512),
                                 (16384, 2048), (20000, 512), (70000, 2048), (200000, 512)])
def test_select_topk(n, k):
    Q = 3
    s = _rand_scores(Q, n, seed=n + k)
    nv = [n, max(0, n - 5), n // 2]
    out = _topk(s, nv, k)
    for i in range(Q):
        checks.check_topk_exact(out[i], s[i, :nv[i]], k)


@pytest.mark.parametrize("n", [3000, 10000])
def test_select_topk_all_equal_and_empty(n):
    s = np.zeros((2, n), np.float32)
    out = _topk(s, [n, 0], 512)
    assert np.array_equal(out[0], np.arange(512))      # ties go to the lowest ids
    assert np.all(out[1] == -1)


@pytest.mark.parametrize("n", [16384, 3001, 700, 20000])
def test_select_topk_col_ids(n):
    """Mapped columns: one round with the ids loaded beside the scores (row
    stride a multiple of 16 or not, 256- and 1024-thread selectors) and the
    multi-round case past 16,384 columns, which maps the ids at the end."""
    Q = 2
    rng = np.random.default_rng(3)
    s = _rand_scores(Q, n, seed=4)
    ids = np.stack([np.sort(rng.choice(1 << 20, n, replace=False)) for _ in range(Q)]).astype(np.int32)
    nv = [n, min(n, 9000) - 1]
    out = _topk(s, nv, 512, ids)
    for i in range(Q):
        checks.check_topk_exact(out[i], s[i, :nv[i]], 512, ids[i, :nv[i]])


@pytest.mark.parametrize("n", [3000, 20000, 70000])
def test_select_topk_extremes(n):
    """Infinities, signed zeros and subnormals among the scores (ordered as
    fp32 values, +0 == -0, ties to the lower id), in one- and multi-round
    selections."""
    Q = 2
    rng = np.random.default_rng(n)
    s = rng.standard_normal((Q, n)).astype(np.float32)
    s[:, ::97] = np.inf
    s[:, 5::89] = -np.inf
    s[:, 7::13] = -0.0
    s[:, 9::17] = 0.0
    s[:, 11::19] = np.float32(1e-40)          # subnormal
    s[1, :] = np.where(s[1, :] > 0, np.float32(3.0), s[1, :])   # a huge tie block
    nv = [n, n - 3]
    out = _topk(s, nv, 512)
    for i in range(Q):
        checks.check_topk_exact(out[i], s[i, :nv[i]], 512)


@pytest.mark.parametrize("n", [1, 300, 512])
def test_select_topk_keep_all(n):
    """At most k valid columns: every one is kept, in id order, mapped
    through col_ids when given."""
    Q = 2
    rng = np.random.default_rng(7)
    s = _rand_scores(Q, max(n, 600), seed=8)
    ids = np.stack([np.sort(rng.choice(1 << 20, s.shape[1], replace=False)) for _ in range(Q)]).astype(np.int32)
    nv = [n, max(0, n - 1)]
    for col in (None, ids):
        out = _topk(s, nv, 512, col)
        for i in range(Q):
            checks.check_topk_exact(out[i], s[i, :nv[i]], 512, None if col is None else ids[i, :nv[i]])


@pytest.mark.parametrize("n", [300000, 16384 * 8 + 5])
def test_block_pool_heavy_ties(n):
    """Scores on a coarse grid (thousands of exact ties at every threshold)
    and an all-equal row: the pool and top-k still follow the (score desc,
    id asc) order in every round of the pyramid."""
    Q = 2
    rng = np.random.default_rng(n)
    s = (np.floor(rng.standard_normal((Q, n)) * 4) / 4).astype(np.float32)
    s[1, :] = 1.0
    nv = [n, n - 7]
    ws = C.workspace(C.CSA2_OP_POOL, Q, n, 2048, DEV)
    pool = torch.empty(Q, 16384, dtype=torch.int32, device=DEV)
    plen = torch.empty(Q, dtype=torch.int64, device=DEV)
    topk = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    C.csa2_block_pool(torch.from_numpy(s).to(DEV), torch.tensor(nv, dtype=torch.int64).to(DEV), n,
                      2048, pool, plen, ws, topk=topk)
    torch.cuda.synchronize()
    for i in range(Q):
        checks.check_pool_exact(checks.host(pool[i]), checks.host(plen[i]), s[i, :nv[i]], 8, 2048)
        checks.check_topk_exact(checks.host(topk[i]), s[i, :nv[i]], 512)
    assert np.array_equal(checks.host(topk[1]), np.arange(512))


@pytest.mark.parametrize("n", [3, 2048, 16384 + 3, 16384 * 8 + 5, 300000])
def test_block_pool(n):
    Q = 2
    s = _rand_scores(Q, n, seed=n)
    nv = [n, max(1, n - 9)]
    ws = C.workspace(C.CSA2_OP_POOL, Q, n, 2048, DEV)
    pool = torch.empty(Q, 16384, dtype=torch.int32, device=DEV)
    plen = torch.empty(Q, dtype=torch.int64, device=DEV)
    topk = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    C.csa2_block_pool(torch.from_numpy(s).to(DEV), torch.tensor(nv, dtype=torch.int64).to(DEV), n,
                      2048, pool, plen, ws, topk=topk)
    torch.cuda.synchronize()
    for i in range(Q):
        checks.check_pool_exact(checks.host(pool[i]), checks.host(plen[i]), s[i, :nv[i]], 8, 2048)
        checks.check_topk_exact(checks.host(topk[i]), s[i, :nv[i]], 512)


def test_select_and_pool_many_queries():
    # more than 64 queries: the selection waits for n_valid before its first
    # loads and the maxima pyramid is built without speculation; ragged
    # visible counts on both sides of the one-round capacity (16,384), an
    # empty row and a full one; the workgroups take the rows last-first
    Q, n = 80, 40000
    s = _rand_scores(Q, n, seed=81)
    rng = np.random.default_rng(82)
    nv = rng.integers(1, n + 1, Q)
    nv[:4] = [n, 0, 16384, 16385]
    nv = [int(x) for x in nv]
    out = _topk(s, nv, 512)
    for i in range(Q):
        if nv[i] == 0:
            assert np.all(out[i] == -1)
        else:
            checks.check_topk_exact(out[i], s[i, :nv[i]], 512)
    nvp = [max(1, x) for x in nv]
    ws = C.workspace(C.CSA2_OP_POOL, Q, n, 2048, DEV)
    pool = torch.empty(Q, 16384, dtype=torch.int32, device=DEV)
    plen = torch.empty(Q, dtype=torch.int64, device=DEV)
    topk = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    C.csa2_block_pool(torch.from_numpy(s).to(DEV), torch.tensor(nvp, dtype=torch.int64).to(DEV), n,
                      2048, pool, plen, ws, topk=topk)
    torch.cuda.synchronize()
    for i in range(Q):
        checks.check_pool_exact(checks.host(pool[i]), checks.host(plen[i]), s[i, :nvp[i]], 8, 2048)
        checks.check_topk_exact(checks.host(topk[i]), s[i, :nvp[i]], 512)


def test_block_pool_small_blocks_and_topk():
    # few blocks, k equal to the block count, heavy ties
    Q, n = 2, 5000
    s = _rand_scores(Q, n, seed=77)
    s[1, :] = 2.0
    ws = C.workspace(C.CSA2_OP_POOL, Q, n, 64, DEV)
    pool = torch.empty(Q, 64 * 8, dtype=torch.int32, device=DEV)
    plen = torch.empty(Q, dtype=torch.int64, device=DEV)
    topk = torch.empty(Q, 64, dtype=torch.int32, device=DEV)
    C.csa2_block_pool(torch.from_numpy(s).to(DEV), torch.tensor([n, n], dtype=torch.int64).to(DEV),
                      n, 64, pool, plen, ws, topk=topk)
    torch.cuda.synchronize()
    for i in range(Q):
        checks.check_pool_exact(checks.host(pool[i]), checks.host(plen[i]), s[i], 8, 64)
        checks.check_topk_exact(checks.host(topk[i]), s[i], 64)


def _swa(nseq, T_swa, seed):
    g = torch.Generator().manual_seed(seed)
    lat = torch.randn(nseq, T_swa, 512, generator=g)
    scale = lat.abs().amax(2) / 448
    codes = (lat / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


@pytest.mark.parametrize("Q,k", [(2, 512), (3, 100), (255, 513), (256, 2048), (300, 64), (260, 1)])
def test_sparse_attend(Q, k):
    """Decode-sized batches take the split-row kernel, 256 queries and more
    the one-workgroup-per-query kernel; both against the oracle."""
    B, N = 2, max(1500, k + 300)
    _, _, _, cache = _build(B, N, 1, seed=31 + Q)
    rng = np.random.default_rng(Q)
    g = torch.Generator().manual_seed(Q)
    q = (torch.randn(Q, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_seq = rng.integers(0, B, Q).astype(np.int32)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(Q)]).astype(np.int32)
    idx[0, ::5] = -1                                  # masked selections
    T_swa = 200
    swa_c, swa_s = _swa(B, T_swa, 9)
    start = rng.integers(0, T_swa, Q).astype(np.int64)   # windows past slot T_swa - 1 wrap
    slen = rng.integers(0, 129, Q).astype(np.int32)
    slen[0] = 128
    start[1 % Q], slen[1 % Q] = T_swa - 1, 128        # wraps after its first row
    slen[-1] = 0                                      # no window at all
    out = torch.empty(Q, 64, 512, device=DEV)
    lse = torch.empty(Q, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_ATTEND, Q, 0, k, DEV)
    C.csa2_sparse_attend(q.to(DEV), torch.from_numpy(q_seq).to(DEV), cache, torch.from_numpy(idx).to(DEV),
                         swa_c.to(DEV), swa_s.to(DEV), torch.from_numpy(start).to(DEV),
                         torch.from_numpy(slen).to(DEV), out, lse, ws)
    torch.cuda.synchronize()
    o, l = checks.host(out), checks.host(lse)
    q64 = checks.bf16_to_f64(q)
    kv_c = checks.host(cache.kv_codes)
    kv_s = checks.host(cache.kv_scales)
    sc_np, ss_np = swa_c.numpy(), swa_s.double().numpy()
    check_q = sorted(set(range(min(Q, 24))) | set(rng.integers(0, Q, 16).tolist()) | {Q - 1})
    for i in check_q:
        b = q_seq[i]
        wc, ws_ = checks.swa_rows(sc_np[b], ss_np[b], int(start[i]), int(slen[i]))
        rows = R.gather_rows(kv_c[b], kv_s[b], idx[i], wc, ws_)
        checks.check_attention(o[i], l[i], q64[i], rows, lse_scale=True)   # rows spread over binades


def _bf16_bits_to_f64(t):
    return checks.host(t.view(torch.int16).to(torch.int32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("Q,dims,split", [(3, 64, True), (1, 64, False), (2, 32, True),
                                          (300, 64, False), (260, 2, False)])
def test_sparse_attend_rope(Q, dims, split):
    """Fused RoPE - attention - inverse RoPE - bf16 cast against the oracle:
    the decode kernel with its split merge (split) or in one workgroup per
    head group (no workspace), and the one-workgroup-per-query kernel (Q >=
    256); positions from 0 to past 2^20 (angles up to 10^6 radians)."""
    B, N, k = 2, 1500, 200
    _, _, _, cache = _build(B, N, 1, seed=71 + Q)
    rng = np.random.default_rng(Q + dims)
    g = torch.Generator().manual_seed(Q + 1)
    q = (torch.randn(Q, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_seq = rng.integers(0, B, Q).astype(np.int32)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(Q)]).astype(np.int32)
    idx[0, ::7] = -1
    T_swa = 200
    swa_c, swa_s = _swa(B, T_swa, 11)
    start = rng.integers(0, T_swa, Q).astype(np.int64)
    slen = rng.integers(0, 129, Q).astype(np.int32)
    pos = rng.integers(0, (1 << 20) + 5000, Q).astype(np.int64)
    pos[0] = 0
    theta = 10000.0
    out = torch.empty(Q, 64, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(Q, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_ATTEND, Q, 0, k, DEV) if split else None
    args = (q.to(DEV), torch.from_numpy(q_seq).to(DEV), cache, torch.from_numpy(idx).to(DEV),
            swa_c.to(DEV), swa_s.to(DEV), torch.from_numpy(start).to(DEV),
            torch.from_numpy(slen).to(DEV))
    C.csa2_sparse_attend_rope(*args, torch.from_numpy(pos).to(DEV), dims, theta, out, lse, ws)
    # no rotation: the plain kernel's fp32 output rounded to bf16, bit for bit
    out0 = torch.empty_like(out)
    C.csa2_sparse_attend_rope(*args, None, 0, theta, out0, None, ws)
    plain = torch.empty(Q, 64, 512, device=DEV)
    C.csa2_sparse_attend(*args, plain, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out0, plain.to(torch.bfloat16))
    o, l = _bf16_bits_to_f64(out), checks.host(lse)
    q64 = checks.bf16_to_f64(q)
    kv_c, kv_s = checks.host(cache.kv_codes), checks.host(cache.kv_scales)
    sc_np, ss_np = swa_c.numpy(), swa_s.double().numpy()
    for i in sorted(set(range(min(Q, 12))) | {Q - 1}):
        b = q_seq[i]
        wc, ws_ = checks.swa_rows(sc_np[b], ss_np[b], int(start[i]), int(slen[i]))
        rows = R.gather_rows(kv_c[b], kv_s[b], idx[i], wc, ws_)
        _, o_ref, lse_ref = R.attend_rope(q64[i], rows, int(pos[i]), dims, theta)
        checks.check_attention_bf16(o[i], l[i], o_ref, lse_ref, R.rope_rotate(q64[i], int(pos[i]), dims, theta), rows,
                                    lse_scale=True)


def test_sparse_attend_wide_trailing_empty_chunks():
    """The one-workgroup-per-query kernel on rows whose selected ids stop
    early (a causal query that sees fewer than k entries: -1 after its last
    id, also -1 inside): against the oracle, and bit for bit the same when
    the id rows are padded with 512 more -1 columns."""
    B, N, Q, k = 2, 1500, 272, 512
    _, _, _, cache = _build(B, N, 1, seed=83)
    rng = np.random.default_rng(83)
    g = torch.Generator().manual_seed(83)
    q = (torch.randn(Q, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_seq = rng.integers(0, B, Q).astype(np.int32)
    idx = np.full((Q, k), -1, dtype=np.int32)
    counts = [0, 1, 2, 63, 64, 65, 127, 128, 129, 200, 448, 449, 511, 512]
    nv = np.array([counts[i % len(counts)] for i in range(Q)])
    for i in range(Q):
        idx[i, :nv[i]] = np.sort(rng.choice(N, nv[i], replace=False))
        if nv[i] > 100 and i % 3 == 0:
            idx[i, 5:70] = -1                       # a whole empty chunk before the last ids
    T_swa = 200
    swa_c, swa_s = _swa(B, T_swa, 13)
    start = rng.integers(0, T_swa, Q).astype(np.int64)
    slen = rng.integers(0, 129, Q).astype(np.int32)
    slen[::5] = 0                                   # some queries without a window
    args = (q.to(DEV), torch.from_numpy(q_seq).to(DEV), cache)
    swa = (swa_c.to(DEV), swa_s.to(DEV), torch.from_numpy(start).to(DEV), torch.from_numpy(slen).to(DEV))
    out = torch.empty(Q, 64, 512, device=DEV)
    lse = torch.empty(Q, 64, device=DEV)
    C.csa2_sparse_attend(*args, torch.from_numpy(idx).to(DEV), *swa, out, lse, None)
    wide = np.concatenate([idx, np.full((Q, 512), -1, dtype=np.int32)], axis=1)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    C.csa2_sparse_attend(*args, torch.from_numpy(wide).to(DEV), *swa, out2, lse2, None)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    o, l = checks.host(out), checks.host(lse)
    q64 = checks.bf16_to_f64(q)
    kv_c, kv_s = checks.host(cache.kv_codes), checks.host(cache.kv_scales)
    sc_np, ss_np = swa_c.numpy(), swa_s.double().numpy()
    for i in sorted(set(range(2 * len(counts))) | {Q - 1}):
        b = q_seq[i]
        wc, ws_ = checks.swa_rows(sc_np[b], ss_np[b], int(start[i]), int(slen[i]))
        rows = R.gather_rows(kv_c[b], kv_s[b], idx[i], wc, ws_)
        if len(rows) == 0:
            assert np.all(o[i] == 0) and np.all(np.isneginf(l[i]))
            continue
        checks.check_attention(o[i], l[i], q64[i], rows, lse_scale=True)


@pytest.mark.parametrize("Q,split", [(2, True), (2, False), (260, False)])
def test_sparse_attend_rising_scores(Q, split):
    """Logits up to a few hundred that grow chunk after chunk (rows ordered
    by their score along the query's direction), so the running softmax
    maximum moves past its slack many times and every rescale path of the
    online softmax runs; heads of odd index see the reverse order (their
    maximum comes first).  Decode kernel with and without its split merge,
    and the one-workgroup-per-query kernel, against the oracle."""
    B, N, k = 1, 1500, 512
    _, _, _, cache = _build(B, N, 1, seed=91)
    rng = np.random.default_rng(91 + Q)
    kv_c, kv_s = checks.host(cache.kv_codes), checks.host(cache.kv_scales)
    K = R.dequant_main_kv(kv_c[0], kv_s[0])                       # [N, 512] fp64
    e_u = int(rng.integers(0, N))
    u = K[e_u]                                                       # the queries' direction
    r = K @ u
    order = np.argsort(r, kind="stable")
    order = order[order != e_u]                                      # the other rows, by r
    r_sd = np.std(r[order])
    idx = np.empty((Q, k), dtype=np.int32)
    q = np.empty((Q, 64, 512))
    sign = np.where(np.arange(64) % 2 == 0, 1.0, -1.0)
    for i in range(Q):
        sel = np.sort(rng.choice(len(order), k, replace=False))      # ranks, ascending
        idx[i] = order[sel]                                          # rows by rising score
        amp = rng.uniform(100.0, 400.0, 64) * sign / (4.0 * r_sd)   # logits over about +-amp
        q[i] = amp[:, None] * u[None, :]
    qb = torch.from_numpy(q).to(torch.bfloat16)
    T_swa = 200
    swa_c, swa_s = _swa(B, T_swa, 17)
    start = rng.integers(0, T_swa, Q).astype(np.int64)
    slen = rng.integers(0, 129, Q).astype(np.int32)
    q_seq = np.zeros(Q, dtype=np.int32)
    out = torch.empty(Q, 64, 512, device=DEV)
    lse = torch.empty(Q, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_ATTEND, Q, 0, k, DEV) if split else None
    C.csa2_sparse_attend(qb.to(DEV), torch.from_numpy(q_seq).to(DEV), cache,
                         torch.from_numpy(idx).to(DEV), swa_c.to(DEV), swa_s.to(DEV),
                         torch.from_numpy(start).to(DEV), torch.from_numpy(slen).to(DEV), out, lse, ws)
    torch.cuda.synchronize()
    o, l = checks.host(out), checks.host(lse)
    q64 = checks.bf16_to_f64(qb)
    sc_np, ss_np = swa_c.numpy(), swa_s.double().numpy()
    for i in sorted(set(range(min(Q, 6))) | {Q - 1}):
        wc, ws_ = checks.swa_rows(sc_np[0], ss_np[0], int(start[i]), int(slen[i]))
        rows = R.gather_rows(kv_c[0], kv_s[0], idx[i], wc, ws_)
        lg = q64[i] @ rows.T
        assert np.abs(lg).max() > 50.0                              # the test's premise
        checks.check_attention(o[i], l[i], q64[i], rows, lse_scale=True)


@pytest.mark.parametrize("Q", [1, 256])
def test_sparse_attend_no_rows(Q):
    _, _, _, cache = _build(1, 64, 1, seed=2)
    q = torch.zeros(Q, 64, 512, dtype=torch.bfloat16, device=DEV)
    idx = torch.full((Q, 8), -1, dtype=torch.int32, device=DEV)
    out = torch.full((Q, 64, 512), 5.0, device=DEV)
    lse = torch.zeros(Q, 64, device=DEV)
    z64 = torch.zeros(Q, dtype=torch.int64, device=DEV)
    z32 = torch.zeros(Q, dtype=torch.int32, device=DEV)
    C.csa2_sparse_attend(q, z32, cache, idx, None, None, z64, z32, out, lse,
                         C.workspace(C.CSA2_OP_ATTEND, Q, 0, 8, DEV))
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isinf(lse)) and torch.all(lse < 0)


def test_check_mode_rejects_bad_indices(monkeypatch):
    """CSA2_CHECK=1: out-of-range device indices are reported as CSA2_EINVAL
    before any kernel reads through them; valid ones pass."""
    B, N, Q, k = 2, 300, 2, 16
    _, _, _, cache = _build(B, N, 1, seed=41)
    q = torch.zeros(Q, 64, 512, dtype=torch.bfloat16, device=DEV)
    q_seq = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    z64 = torch.zeros(Q, dtype=torch.int64, device=DEV)
    z32 = torch.zeros(Q, dtype=torch.int32, device=DEV)
    out = torch.empty(Q, 64, 512, device=DEV)
    ws = C.workspace(C.CSA2_OP_ATTEND, Q, 0, k, DEV)
    idx = torch.arange(Q * k, dtype=torch.int32, device=DEV).reshape(Q, k)
    monkeypatch.setenv("CSA2_CHECK", "1")
    C.csa2_sparse_attend(q, q_seq, cache, idx, None, None, z64, z32, out, None, ws)
    bad = idx.clone()
    bad[1, 3] = N                                     # one past the cache capacity
    with pytest.raises(C.Csa2Error, match="idx"):
        C.csa2_sparse_attend(q, q_seq, cache, bad, None, None, z64, z32, out, None, ws)
    qi, w = _scores_inputs(Q, 42)
    cand = torch.zeros(Q, 40, dtype=torch.int32, device=DEV)
    cand[0, 39] = -5                                  # outside [0, cap) but past n_vis[0]: ignored
    nv = torch.tensor([39, 40], dtype=torch.int64, device=DEV)
    sc = torch.empty(Q, 40, device=DEV)
    C.csa2_index_score(qi.to(DEV), w.to(DEV), q_seq, nv, cand, 40, cache, sc)
    cand[1, 10] = N
    with pytest.raises(C.Csa2Error, match="cand"):
        C.csa2_index_score(qi.to(DEV), w.to(DEV), q_seq, nv, cand, 40, cache, sc)
    # a sequence id at the cache's batch count (2 sequences): caught by the
    # check before any kernel is launched
    seq_bad = torch.tensor([0, B], dtype=torch.int32, device=DEV)
    with pytest.raises(C.Csa2Error, match="q_seq"):
        C.csa2_sparse_attend(q, seq_bad, cache, idx, None, None, z64, z32, out, None, ws)
    with pytest.raises(C.Csa2Error, match="q_seq"):
        C.csa2_index_score(qi.to(DEV), w.to(DEV), seq_bad, nv, None, 40, cache, sc)
    torch.cuda.synchronize()


def test_c0_step():
    from long_context_sparse_csa2_amd.pipeline import Step
    step = Step(synth.WORKLOADS["c0"], DEV)
    step.run(keep=True)
    torch.cuda.synchronize()
    checks.check_step(step)


def test_determinism():
    from long_context_sparse_csa2_amd.pipeline import Step
    step = Step(synth.scaled(synth.WORKLOADS["c2"], B=2, T=40000), DEV)
    step.run(keep=True)
    a = [t.clone() for t in step.out] + [x.clone() for x in step.idx_per_layer]
    step.run(keep=True)
    b = list(step.out) + list(step.idx_per_layer)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("split_first", [True, False])
def test_graph_replay_matches_eager(split_first):
    """The step captured as HIP graphs (as bench.py replays it: one graph,
    or the scan apart from the rest) gives the eager result on every replay,
    with eager work in between."""
    from long_context_sparse_csa2_amd.pipeline import Step
    step = Step(synth.scaled(synth.WORKLOADS["c2"], B=2, T=50000), DEV)
    step.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in step.out] + [step.pool.clone(), step.idx.clone()]
    graphs = step.capture(split_first=split_first)
    for rep in range(3):
        for t in step.out:
            t.zero_()                     # eager work between replays
        step.pool.fill_(-5)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        got = list(step.out) + [step.pool, step.idx]
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
