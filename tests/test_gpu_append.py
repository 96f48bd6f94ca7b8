"""Decode-time append (state block of the V4 KV layout, Fig. 6 of the
DeepSeek-V4 page): tokens appended one at a time through the C ABI against
the oracle's append_token, then one decode query attending over the
appended cache and the SWA ring."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_csa2_amd as C
from oracle import csa2_ref as R
from tests import checks

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _tokens(B, T, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, T, 512, generator=g) * torch.exp(torch.empty(B, T, 1).uniform_(-6, 4, generator=g))
    z = torch.randn(B, T, 512, generator=g) * 2
    sw = torch.randn(B, T, 512, generator=g) * torch.exp(torch.empty(B, T, 1).uniform_(-8, 8, generator=g))
    sw[0, 2] = 0.0                                    # an all-zero SWA row
    return h.to(torch.bfloat16), z.to(torch.bfloat16), sw.to(torch.bfloat16)


@pytest.mark.parametrize("m,W,cap", [(1, 8, 64), (2, 8, 64), (4, 128, 64), (2, 8, 3)])
def test_decode_append(m, W, cap):
    """B = 3 sequences at different token counts (sequence 0 gets 5 extra
    tokens first); every entry, tail token, SWA ring slot and geometry output
    against the oracle; cap = 3 drops the entries past the cache."""
    B, T = 3, 13 if m < 4 else 23
    h, z, sw = _tokens(B, T + 5, 40 + m)
    w_ik = (torch.randn(128, 512, generator=torch.Generator().manual_seed(7)) / math.sqrt(512)).to(torch.bfloat16)
    cache = C.Cache(B, cap, DEV)
    for a in cache.arrays().values():
        a.fill_(0xAB)
    st = C.State(B, m, W, DEV)
    hd, zd, swd, wd = h.to(DEV), z.to(DEV), sw.to(DEV), w_ik.to(DEV)
    n_vis = torch.zeros(B, dtype=torch.int64, device=DEV)
    s0 = torch.zeros(B, dtype=torch.int64, device=DEV)
    sl = torch.zeros(B, dtype=torch.int32, device=DEV)
    counts = [0] * B
    # sequence 0 alone first (a one-sequence view of the state and cache)
    for t in range(5):
        C.csa2_decode_append(hd[0:1, t].contiguous(), zd[0:1, t].contiguous() if m > 1 else None,
                             swd[0:1, t].contiguous(), wd, cache.view(0, 1), st.view(0, 1))
        counts[0] += 1
    for t in range(T):
        rows = [counts[b] for b in range(B)]
        hn = torch.stack([hd[b, rows[b]] for b in range(B)])
        zn = torch.stack([zd[b, rows[b]] for b in range(B)]) if m > 1 else None
        sn = torch.stack([swd[b, rows[b]] for b in range(B)])
        C.csa2_decode_append(hn, zn, sn, wd, cache, st, n_vis, s0, sl)
        for b in range(B):
            counts[b] += 1
        torch.cuda.synchronize()
        got = (checks.host(n_vis), checks.host(s0), checks.host(sl))
        for b in range(B):
            want = R.decode_geometry(counts[b], m, W)
            assert (int(got[0][b]), int(got[1][b]), int(got[2][b])) == want, (t, b)
    assert checks.host(st.n_tok).tolist() == counts
    w64 = checks.bf16_to_f64(w_ik)
    for b in range(B):
        n_tok = counts[b]
        hb, zb, sb = checks.bf16_to_f64(h[b, :n_tok]), checks.bf16_to_f64(z[b, :n_tok]), checks.bf16_to_f64(sw[b, :n_tok])
        n = n_tok // m
        kept = min(n, cap)
        kv_c, kv_s = checks.host(cache.kv_codes[b]), checks.host(cache.kv_scales[b])
        ik_c, ik_s = checks.host(cache.ik_codes[b]), checks.host(cache.ik_scales[b])
        x = R.compress(hb[:kept * m], None if m == 1 else zb[:kept * m], m)
        hmax = np.abs(hb[:kept * m]).reshape(-1, m, 512).max(1)
        checks.check_main_kv(x, m, kv_c[:kept], kv_s[:kept], hmax)
        checks.check_indexer_k(kv_c[:kept], kv_s[:kept], w64, ik_c[:kept], ik_s[:kept])
        assert np.all(kv_c[kept:] == 0xAB) and np.all(ik_s[kept:] == 0xAB)   # nothing past the count / cap
        if m > 1:
            r = n_tok - n * m
            assert np.array_equal(checks.host(st.tail_h[b, :r].view(torch.int16)),
                                  h[b, n * m:n_tok].view(torch.int16).numpy())
            assert np.array_equal(checks.host(st.tail_z[b, :r].view(torch.int16)),
                                  z[b, n * m:n_tok].view(torch.int16).numpy())
        # ring: slot t % W holds token t's row for the last W tokens
        slots = np.arange(max(0, n_tok - W), n_tok) % W
        checks.check_swa_rows(checks.host(st.swa_codes[b])[slots], checks.host(st.swa_scale[b])[slots],
                              sb[max(0, n_tok - W):n_tok])


def test_decode_loop_attends_over_ring():
    """m = 1, W = 8: 20 appended tokens, then one query per sequence scoring
    its visible entries and attending over all of them plus the SWA ring
    window (wrapped), with the geometry the append wrote."""
    B, T, W = 2, 20, 8
    h, _, sw = _tokens(B, T, 77)
    w_ik = (torch.randn(128, 512, generator=torch.Generator().manual_seed(8)) / math.sqrt(512)).to(torch.bfloat16)
    cache = C.Cache(B, 32, DEV)
    st = C.State(B, 1, W, DEV)
    n_vis = torch.zeros(B, dtype=torch.int64, device=DEV)
    s0 = torch.zeros(B, dtype=torch.int64, device=DEV)
    sl = torch.zeros(B, dtype=torch.int32, device=DEV)
    hd, swd, wd = h.to(DEV), sw.to(DEV), w_ik.to(DEV)
    for t in range(T):
        C.csa2_decode_append(hd[:, t].contiguous(), None, swd[:, t].contiguous(), wd, cache, st,
                             n_vis, s0, sl)
    g = torch.Generator().manual_seed(9)
    q = (torch.randn(B, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_seq = torch.arange(B, dtype=torch.int32, device=DEV)
    idx = torch.arange(T, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    out = torch.empty(B, 64, 512, device=DEV)
    lse = torch.empty(B, 64, device=DEV)
    ws = C.workspace(C.CSA2_OP_ATTEND, B, 0, T, DEV)
    C.csa2_sparse_attend(q.to(DEV), q_seq, cache, idx, st.swa_codes, st.swa_scale, s0, sl, out, lse, ws)
    torch.cuda.synchronize()
    assert checks.host(n_vis).tolist() == [T] * B
    assert checks.host(s0).tolist() == [(T - W) % W] * B and checks.host(sl).tolist() == [W] * B
    o, l = checks.host(out), checks.host(lse)
    for b in range(B):
        kv_c, kv_s = checks.host(cache.kv_codes[b]), checks.host(cache.kv_scales[b])
        wc, wsc = checks.swa_rows(checks.host(st.swa_codes[b]), checks.host(st.swa_scale[b]).astype(np.float64),
                                  (T - W) % W, W)
        checks.check_swa_rows(wc, wsc.astype(np.float32), checks.bf16_to_f64(sw[b, T - W:T]))
        rows = R.gather_rows(kv_c, kv_s, np.arange(T), wc, wsc)
        checks.check_attention(o[b], l[b], checks.bf16_to_f64(q[b]), rows, lse_scale=True)   # rows spread over binades
