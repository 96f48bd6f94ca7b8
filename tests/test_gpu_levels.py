"""csa2_index_score_levels + csa2_select_attend_levels (the scan writes the
selection's lowest maxima levels) against csa2_index_score +
csa2_select_attend (the selection's own maxima pass) on the same inputs,
through the C ABI: scores, every maxima group of every query, the top-k
ids, the pool and the attention outputs, all bit for bit.  The shapes cover
the scan's interleaved and contiguous layouts, one and two levels, a level
count the scan epilogue does not produce (three levels: the maxima pass
runs inside the levels call) and a scan of one tile per wave (no tile
pairs), with ragged visible counts."""
import numpy as np
import pytest
import torch

import long_context_sparse_csa2_amd as C

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SEL_CAP = 16384


def _groups(n, lvl):
    return -(-n // 8 ** lvl)


def _layout(Q, n_cols, mode):
    """Level offsets and row strides (uint32 units) of the selection's
    maxima pyramid in its workspace."""
    L = 0
    while _groups(n_cols, L) > SEL_CAP:
        L += 1
    L = max(L, mode)
    off, lv = 0, {}
    for l in range(1, L + 1):
        stride = -(-_groups(n_cols, l) // 16) * 16
        lv[l] = (off, stride)
        off += Q * stride
    return lv


def _cache(B, N, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    cache = C.Cache(B, N, DEV)
    cache.ik_codes.random_(0, 256, generator=g)
    cache.ik_scales.random_(118, 131, generator=g)            # E8M0 2^-9 .. 2^3
    cache.kv_codes.random_(0, 256, generator=g)
    cache.kv_scales.random_(0x28, 0x48, generator=g)          # E4M3 in [2^-2, 2^2)
    return cache


def _inputs(Q, B, seed):
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    q_idx = torch.randn(Q, 32, 128, device=DEV, generator=g).to(torch.bfloat16)
    w = torch.rand(Q, 32, device=DEV, generator=g)
    q = (torch.randn(Q, 64, 512, device=DEV, generator=g) / 22.6).to(torch.bfloat16)
    q_seq = (torch.arange(Q, device=DEV) % B).to(torch.int32)
    T = 256
    swa_c = torch.randint(0, 0x77, (B, T, 512), device=DEV, generator=g, dtype=torch.int32).to(torch.uint8)
    swa_s = torch.full((B, T), 0.01, device=DEV)
    start = (torch.arange(Q, device=DEV, dtype=torch.int64) * 37) % T
    slen = torch.full((Q,), 128, dtype=torch.int32, device=DEV)
    return q_idx, w, q, q_seq, swa_c, swa_s, start, slen


@pytest.mark.parametrize("Q,n_cols,nb,fp4q", [
    (4, 1 << 20, 2048, False),      # 1M decode: 32 tiles per wave, interleaved slices, 2 levels
    (8, 300001, 0, False),          # 16 tiles per wave, interleaved, 2 levels, ragged tail
    (32, 65536, 0, True),           # 64K decode, contiguous chunks, 1 level, MXFP4 query
    (2, (1 << 21) + 77, 2048, False),  # 3 levels: the maxima pass inside the levels call
    (5, 5000, 0, False),            # one tile per wave: the maxima pass inside the levels call
])
def test_levels_equal_separate(Q, n_cols, nb, fp4q):
    B, k = 2, 512
    cache = _cache(B, n_cols, seed=n_cols % 997 + Q)
    q_idx, w, q, q_seq, swa_c, swa_s, start, slen = _inputs(Q, B, seed=Q)
    nv_h = [n_cols - 13 * i - (i % 3) for i in range(Q)]
    nv_h[-1] = min(n_cols, 1000 + 5 * Q)                 # a short row: partial groups at every level
    nv = torch.tensor(nv_h, dtype=torch.int64, device=DEV)
    mode = 1 if nb else 0
    op = C.CSA2_OP_POOL_ATTEND if nb else C.CSA2_OP_SELECT_ATTEND
    res = {}
    for levels in (False, True):
        scores = torch.full((Q, n_cols), -5.0, device=DEV)
        idx = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
        pool = torch.full((Q, max(nb, 1) * 8), -9, dtype=torch.int32, device=DEV) if nb else None
        plen = torch.full((Q,), -9, dtype=torch.int64, device=DEV) if nb else None
        out = torch.empty(Q, 64, 512, device=DEV)
        lse = torch.empty(Q, 64, device=DEV)
        ws = C.workspace(op, Q, n_cols, k, DEV)
        ws.fill_(0xAB)                                   # no group may keep this filler
        if levels:
            C.csa2_index_score_levels(q_idx, w, q_seq, nv, n_cols, cache, scores, ws, n_blocks=nb,
                                      fp4q=fp4q)
        else:
            C.csa2_index_score(q_idx, w, q_seq, nv, None, n_cols, cache, scores, fp4q=fp4q)
        C.csa2_select_attend(scores, nv, None, n_cols, k, idx, q, q_seq, cache, swa_c, swa_s,
                             start, slen, out, lse, ws, n_blocks=nb, pool=pool, pool_len=plen,
                             levels=levels)
        torch.cuda.synchronize()
        res[levels] = (scores, idx, pool, plen, out, lse, ws.view(torch.int32))
    a, b = res[False], res[True]
    for i in range(Q):
        assert torch.equal(a[0][i, :nv_h[i]], b[0][i, :nv_h[i]]), f"scores of query {i}"
    for l, (off, stride) in _layout(Q, n_cols, mode).items():
        for i in range(Q):
            g = _groups(nv_h[i], l)
            la = a[6][off + i * stride: off + i * stride + g]
            lb = b[6][off + i * stride: off + i * stride + g]
            assert torch.equal(la, lb), f"level {l} of query {i}"
    assert torch.equal(a[1], b[1])
    if nb:
        assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])
    assert torch.equal(a[4], b[4]) and torch.equal(a[5], b[5])
    assert int((b[1] >= 0).sum()) == sum(min(k, n) for n in nv_h)


def test_levels_validation():
    """Errors of the two entry points that need no kernel to run."""
    Q, n = 2, 4096
    cache = _cache(1, n, seed=3)
    q_idx, w, q, q_seq, swa_c, swa_s, start, slen = _inputs(Q, 1, seed=3)
    nv = torch.full((Q,), n, dtype=torch.int64, device=DEV)
    scores = torch.empty(Q, n, device=DEV)
    small = torch.empty(256, dtype=torch.uint8, device=DEV)     # a pool needs one level: 4 KB
    with pytest.raises(C.Csa2Error, match="CSA2_EWORKSPACE"):
        C.csa2_index_score_levels(q_idx, w, q_seq, nv, n, cache, scores, small, n_blocks=2048)
    ws = C.workspace(C.CSA2_OP_SELECT_ATTEND, Q, n, 512, DEV)
    idx = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    ids = torch.zeros(Q, n, dtype=torch.int32, device=DEV)
    out = torch.empty(Q, 64, 512, device=DEV)
    with pytest.raises(C.Csa2Error, match="CSA2_EINVAL"):
        C.csa2_select_attend(scores, nv, ids, n, 512, idx, q, q_seq, cache, swa_c, swa_s, start,
                             slen, out, None, ws, levels=True)


@pytest.mark.parametrize("Q,n_cols", [(512, 200000), (64, 1 << 19), (300, 70000)])
def test_topk_levels_equal_separate(Q, n_cols):
    """csa2_index_score_levels + csa2_select_topk_levels against
    csa2_index_score + csa2_select_topk (the prefill path, many queries with
    causal visible counts): scores, maxima groups and top-k ids bit for bit."""
    B, k = 1, 512
    cache = _cache(B, n_cols, seed=Q + 11)
    q_idx, w, *_ = _inputs(Q, B, seed=Q + 12)
    q_seq = torch.zeros(Q, dtype=torch.int32, device=DEV)
    nv_h = [max(1, n_cols - (Q - 1 - i) * (n_cols // Q) - (i % 5)) for i in range(Q)]
    nv = torch.tensor(nv_h, dtype=torch.int64, device=DEV)
    res = {}
    for levels in (False, True):
        scores = torch.full((Q, n_cols), -5.0, device=DEV)
        idx = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
        ws = C.workspace(C.CSA2_OP_TOPK, Q, n_cols, k, DEV)
        ws.fill_(0xAB)
        if levels:
            C.csa2_index_score_levels(q_idx, w, q_seq, nv, n_cols, cache, scores, ws)
        else:
            C.csa2_index_score(q_idx, w, q_seq, nv, None, n_cols, cache, scores)
        C.csa2_select_topk(scores, nv, None, n_cols, k, idx, ws, levels=levels)
        torch.cuda.synchronize()
        res[levels] = (scores, idx, ws.view(torch.int32))
    a, b = res[False], res[True]
    for i in range(Q):
        assert torch.equal(a[0][i, :nv_h[i]], b[0][i, :nv_h[i]]), f"scores of query {i}"
    for l, (off, stride) in _layout(Q, n_cols, 0).items():
        for i in range(Q):
            g = _groups(nv_h[i], l)
            assert torch.equal(a[2][off + i * stride: off + i * stride + g],
                               b[2][off + i * stride: off + i * stride + g]), f"level {l} of query {i}"
    assert torch.equal(a[1], b[1])
