"""csa2_select_attend (selection fused with the attention) against the
separate calls on the same inputs, through the C ABI: the selection
outputs (top-k ids, pool, pool length) bit for bit, the attention against
the fp64 oracle over the selected rows (and against the separate
attention call where both use the same row splits)."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_csa2_amd as C
from oracle import csa2_ref as R
from tests import checks
from tests.test_gpu_kernels import _build, _swa

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(Q, N, n_cols, seed, pool_ids=False):
    B = 2
    _, _, _, cache = _build(B, N, 1, seed=seed)
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    scores = (torch.rand(Q, n_cols, generator=g) * 50).float()
    scores[:, ::37] = scores[:, 3:4]                     # ties
    q = (torch.randn(Q, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_seq = torch.from_numpy(rng.integers(0, B, Q).astype(np.int32))
    T_swa = 160
    swa_c, swa_s = _swa(B, T_swa, seed + 1)
    start = torch.from_numpy(rng.integers(0, T_swa, Q).astype(np.int64))
    slen = torch.from_numpy(rng.integers(0, 129, Q).astype(np.int32))
    slen[0] = 128
    start[1 % Q], slen[1 % Q] = T_swa - 1, 128           # a window that wraps
    slen[-1] = 0                                          # and none at all
    ids = None
    if pool_ids:
        ids = torch.from_numpy(np.stack([np.sort(rng.choice(N, n_cols, replace=False))
                                         for _ in range(Q)]).astype(np.int32))
    return dict(cache=cache, scores=scores.to(DEV), q=q.to(DEV), q_seq=q_seq.to(DEV),
                swa_c=swa_c.to(DEV), swa_s=swa_s.to(DEV), start=start.to(DEV), slen=slen.to(DEV),
                ids=None if ids is None else ids.to(DEV), B=B, N=N)


def _check_rows(c, i, idx_row, o, l):
    b = int(c["q_seq"][i])
    kv_c, kv_s = checks.host(c["cache"].kv_codes[b]), checks.host(c["cache"].kv_scales[b])
    wc, ws_ = checks.swa_rows(checks.host(c["swa_c"][b]), checks.host(c["swa_s"][b]).astype(np.float64),
                              int(c["start"][i]), int(c["slen"][i]))
    rows = R.gather_rows(kv_c, kv_s, idx_row, wc, ws_)
    if rows.shape[0] == 0:
        assert np.all(o == 0) and np.all(np.isneginf(l))
        return
    checks.check_attention(o, l, checks.bf16_to_f64(c["q"][i].cpu()), rows, lse_scale=True)


@pytest.mark.parametrize("Q,n_cols,k,pool_ids", [(4, 16384, 512, True), (3, 16384, 512, False),
                                                 (5, 3000, 100, True), (2, 65536, 512, False),
                                                 (7, 700, 512, False), (1, 20000, 2048, True),
                                                 (11, 3000, 300, True), (24, 4096, 512, False)])
def test_select_attend_topk(Q, n_cols, k, pool_ids):
    """One chunk per workgroup while the workgroups fit the CUs; Q = 7, 11
    and 24 take 2, 2 and 5 consecutive chunks per workgroup (11 and 24 with
    a workgroup whose chunks are main rows followed by SWA rows)."""
    c = _case(Q, max(4096, n_cols + 100), n_cols, seed=Q * 7 + k, pool_ids=pool_ids)
    nv = torch.tensor([n_cols - 3 * i for i in range(Q)], dtype=torch.int64)
    nv[-1] = min(n_cols, 300) if Q > 1 else nv[-1]          # fewer valid columns than k
    nv = nv.to(DEV)
    idx_f = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
    out_f = torch.empty(Q, 64, 512, device=DEV)
    lse_f = torch.empty(Q, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_SELECT_ATTEND, Q, n_cols, k, DEV)
    C.csa2_select_attend(c["scores"], nv, c["ids"], n_cols, k, idx_f, c["q"], c["q_seq"], c["cache"],
                         c["swa_c"], c["swa_s"], c["start"], c["slen"], out_f, lse_f, ws)
    # the separate calls
    idx_s = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    C.csa2_select_topk(c["scores"], nv, c["ids"], n_cols, k, idx_s,
                       C.workspace(C.CSA2_OP_TOPK, Q, n_cols, k, DEV))
    out_s = torch.empty(Q, 64, 512, device=DEV)
    lse_s = torch.empty(Q, 64, device=DEV)
    C.csa2_sparse_attend(c["q"], c["q_seq"], c["cache"], idx_s, c["swa_c"], c["swa_s"], c["start"],
                         c["slen"], out_s, lse_s, C.workspace(C.CSA2_OP_ATTEND, Q, 0, k, DEV))
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s)
    idx = checks.host(idx_f)
    o, l = checks.host(out_f), checks.host(lse_f)
    for i in range(Q):
        _check_rows(c, i, idx[i], o[i], l[i])
    if Q <= 4 and k == 512:                                 # same row splits on both paths
        assert float((out_f - out_s).abs().max()) <= 1e-6 * float(out_s.abs().max())
        assert float((lse_f - lse_s).abs().max()) <= 1e-6 * max(1.0, float(lse_s.abs().max()))


@pytest.mark.parametrize("Q,n", [(3, 300000), (2, 16384 * 8 + 5), (3, 5000)])
def test_select_attend_pool(Q, n):
    c = _case(Q, n, n, seed=n % 1000 + Q)
    nv = torch.tensor([n - 11 * i for i in range(Q)], dtype=torch.int64, device=DEV)
    k, nb = 512, 2048
    idx_f = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
    pool_f = torch.full((Q, nb * 8), -9, dtype=torch.int32, device=DEV)
    plen_f = torch.full((Q,), -9, dtype=torch.int64, device=DEV)
    out_f = torch.empty(Q, 64, 512, device=DEV)
    lse_f = torch.empty(Q, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_POOL_ATTEND, Q, n, k, DEV)
    C.csa2_select_attend(c["scores"], nv, None, n, k, idx_f, c["q"], c["q_seq"], c["cache"],
                         c["swa_c"], c["swa_s"], c["start"], c["slen"], out_f, lse_f, ws,
                         n_blocks=nb, pool=pool_f, pool_len=plen_f)
    idx_s = torch.empty(Q, k, dtype=torch.int32, device=DEV)
    pool_s = torch.empty(Q, nb * 8, dtype=torch.int32, device=DEV)
    plen_s = torch.empty(Q, dtype=torch.int64, device=DEV)
    C.csa2_block_pool(c["scores"], nv, n, nb, pool_s, plen_s, C.workspace(C.CSA2_OP_POOL, Q, n, nb, DEV),
                      topk=idx_s)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s) and torch.equal(pool_f, pool_s) and torch.equal(plen_f, plen_s)
    s = checks.host(c["scores"])
    idx, nvh = checks.host(idx_f), checks.host(nv)
    o, l = checks.host(out_f), checks.host(lse_f)
    for i in range(Q):
        checks.check_topk_exact(idx[i], s[i, :nvh[i]], k)
        checks.check_pool_exact(checks.host(pool_f[i]), checks.host(plen_f[i]), s[i, :nvh[i]], 8, nb)
        _check_rows(c, i, idx[i], o[i], l[i])


def test_select_attend_empty_rows():
    """A query with no valid column and no SWA row: ids all -1, output 0,
    lse -inf; the other query is unaffected."""
    c = _case(2, 4096, 2000, seed=5)
    c["slen"][0] = 0
    nv = torch.tensor([0, 2000], dtype=torch.int64, device=DEV)
    idx = torch.full((2, 512), -9, dtype=torch.int32, device=DEV)
    out = torch.full((2, 64, 512), 7.0, device=DEV)
    lse = torch.empty(2, 64, device=DEV)
    C.csa2_select_attend(c["scores"], nv, None, 2000, 512, idx, c["q"], c["q_seq"], c["cache"],
                         c["swa_c"], c["swa_s"], c["start"], c["slen"], out, lse,
                         C.workspace(C.CSA2_OP_SELECT_ATTEND, 2, 2000, 512, DEV))
    torch.cuda.synchronize()
    assert torch.all(idx[0] == -1)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    h = checks.host(idx)
    checks.check_topk_exact(h[1], checks.host(c["scores"])[1, :2000], 512)
    _check_rows(c, 1, h[1], checks.host(out[1]), checks.host(lse[1]))
