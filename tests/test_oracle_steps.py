"""Pins of each oracle step against closed forms, special cases, invariants
and brute force on tiny inputs.  Each test is chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule) fails it."""
import json
import math
import os
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import csa2_ref as R
from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ a1
def test_compress_m1_identity():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((6, 512))
    assert np.array_equal(R.compress(h, None, 1), h)


def test_compress_special_cases():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((8, 512))
    # constant logits -> plain mean of each pair
    z = np.full((8, 512), 0.7)
    assert np.allclose(R.compress(h, z, 2), h.reshape(4, 2, 512).mean(1), rtol=0, atol=1e-15)
    # a dominant logit picks its row
    z = np.zeros((8, 512))
    z[1::2] = 800.0
    assert np.allclose(R.compress(h, z, 2), h[1::2], rtol=0, atol=0)
    # per-channel weights: channel c uses its own logit column
    z = rng.standard_normal((8, 512)) * 3
    x = R.compress(h, z, 4)
    w = scipy.special.softmax(z.reshape(2, 4, 512), axis=1)
    assert np.allclose(x, (w * h.reshape(2, 4, 512)).sum(1), rtol=1e-14, atol=1e-14)
    # convex combination: inside the per-channel range of its rows
    hh = h.reshape(2, 4, 512)
    assert np.all(x <= hh.max(1) + 1e-12) and np.all(x >= hh.min(1) - 1e-12)


def test_compress_v4_worked_example():
    g = json.load(open(os.path.join(GOLD, "v4_pooling_example.json")))
    v = np.array(g["vectors"])                       # 4 tokens, 2 channels
    w = np.array(g["printed_weights"])
    z = np.repeat(np.log(w)[:, None], 2, axis=1)     # softmax(log w) = w (sum w = 1)
    x = R.compress(v, z, 4)
    assert np.allclose(x[0], g["printed_entry"], atol=1e-12)
    # the printed weights are not the softmax of the printed logits
    true = scipy.special.softmax(np.array(g["printed_logits"]))
    assert not np.allclose(true, w, atol=0.01)


# ------------------------------------------------------------------ a2
def test_main_kv_quant_exact_when_representable():
    rng = np.random.default_rng(3)
    n = 64
    sc = rng.integers(0x08, 0x7F, size=(n, 32))               # normal E4M3 scales
    codes = rng.integers(0, 16, size=(n, 512)).astype(np.uint8)
    codes[:, ::16] = 0x7                                        # group max = 6 * s
    x = (F.e2m1_value(codes).reshape(n, 32, 16) * F.e4m3fn_value(sc)[:, :, None]).reshape(n, 512)
    c, s = R.quant_main_kv(x)
    assert np.array_equal(s, sc)
    assert np.array_equal(R.dequant_main_kv(c, s), x)
    # the largest magnitude the format holds (report section 2.4.4)
    x = np.zeros((1, 512))
    x[0, 5] = -2688.0
    c, s = R.quant_main_kv(x)
    assert R.dequant_main_kv(c, s)[0, 5] == -2688.0


def test_main_kv_quant_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 512)) * np.exp(rng.uniform(-6, 6, (8, 1)))
    c, s = R.quant_main_kv(x)
    allsc = F.e4m3fn_value(np.arange(0x7F))
    e2 = F.e2m1_value(np.arange(16))
    for j in range(8):
        for g in range(32):
            grp = x[j, 16 * g:16 * g + 16]
            a = np.abs(grp).max() / 6
            # scale: nearest E4M3 value to max/6 (tie -> even code)
            d = np.abs(allsc - a)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert s[j, g] == want
            sv = allsc[want]
            nib = F.unpack_nibbles(c[j])[16 * g:16 * g + 16]
            for ch in range(16):
                r = grp[ch] / sv
                dd = np.abs(np.clip(r, -6, 6) - e2)
                assert dd[nib[ch]] == dd.min()
                assert (nib[ch] >= 8) == (grp[ch] < 0)


def test_main_kv_quant_zero_group():
    x = np.zeros((2, 512))
    x[1, :16] = 1e-6                       # max/6 rounds to E4M3 zero
    c, s = R.quant_main_kv(x)
    assert np.all(c == 0) and np.all(s == 0)


# ------------------------------------------------------------------ a3
def test_projection_orientation():
    rng = np.random.default_rng(5)
    xhat = rng.standard_normal((3, 512))
    w = rng.standard_normal((128, 512))
    k = R.project_indexer_k(xhat, w)
    assert k.shape == (3, 128)
    # output dim d reads row d of w
    assert np.isclose(k[2, 7], sum(w[7, c] * xhat[2, c] for c in range(512)), rtol=1e-12)


def test_mxfp4_special_cases():
    k = np.zeros((4, 128))
    k[0, :32] = 3.0          # floor(log2 3) = 1 -> X = 2^-1, 3 / X = 6: exact
    k[0, 32:64] = -1.0       # X = 2^-2, -4: exact
    k[1, :32] = 8.0          # power of two: X = 2, 4: exact
    k[1, 32:64] = 7.99       # X = 1, 7.99 clips to 6
    k[2, :] = np.arange(128) / 16.0
    c, s = R.quant_mxfp4(k)
    d = R.dequant_mxfp4(c, s)
    assert np.all(d[0, :32] == 3.0) and np.all(d[0, 32:64] == -1.0)
    assert s[0, 0] == 126 and s[0, 1] == 125
    assert np.all(d[1, :32] == 8.0) and s[1, 0] == 128
    assert np.all(d[1, 32:64] == 6.0)
    assert s[3, 0] == 0 and np.all(c[3] == 0)                 # all-zero block
    # every element is a nearest representable value of k / X
    for g in range(4):
        X = F.e8m0_value(s[2, g])
        blk = k[2, 32 * g:32 * g + 32]
        assert X == 2.0 ** (math.floor(math.log2(np.abs(blk).max())) - 2)
        e2 = F.e2m1_value(np.arange(16))
        for ch, nib in enumerate(F.unpack_nibbles(c[2])[32 * g:32 * g + 32]):
            dd = np.abs(np.clip(blk[ch] / X, -6, 6) - e2)
            assert dd[nib] == dd.min()


# ------------------------------------------------------------------ a4
def _score_loops(q, w, k):
    out = []
    for j in range(k.shape[0]):
        tot = 0.0
        for h in range(q.shape[0]):
            dot = 0.0
            for c in range(q.shape[1]):
                dot += q[h, c] * k[j, c]
            tot += w[h] * (dot if dot > 0 else 0.0)
        out.append(tot)
    return np.array(out)


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((32, 128))
    w = rng.uniform(0, 1, 32)
    k = rng.standard_normal((5, 128))
    assert np.allclose(R.index_scores(q, w, k), _score_loops(q, w, k), rtol=1e-12)


def test_scores_identities():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((32, 128))
    w = rng.uniform(0, 1, 32)
    k = rng.standard_normal((40, 128))
    s = R.index_scores(q, w, k)
    assert np.all(s >= 0)
    # relu(x) - relu(-x) = x: the difference is the plain weighted dot
    lin = (k @ q.T) @ w
    assert np.allclose(s - R.index_scores(-q, w, k), lin, rtol=1e-10, atol=1e-10)
    # one head with unit weight is relu(q_h . k)
    e = np.zeros(32); e[9] = 1.0
    assert np.allclose(R.index_scores(q, e, k), np.maximum(k @ q[9], 0), rtol=1e-13)
    # positive homogeneity in q and linearity in w
    assert np.allclose(R.index_scores(2.5 * q, w, k), 2.5 * s, rtol=1e-13)
    assert np.allclose(R.index_scores(q, 3 * w, k), 3 * s, rtol=1e-13)


# ------------------------------------------------------------------ f1
def test_fp4q_worked_example():
    """MXFP4 query (report section 2.4.4; OCP MX rule), values worked by
    hand: X = 2^(floor(log2 amax) - 2), RNE to E2M1 with ties to the even
    code, saturation at 6."""
    q = np.zeros((32, 128))
    # head 3, block 1: amax 7 -> X = 1 (byte 127)
    q[3, 32:39] = [5.0, -2.6, 0.3, 0.25, 7.0, -0.1, 1.25]
    # head 0, block 0: amax 0.75 -> X = 2^-3 (byte 124); 0.0375 / X = 0.3 -> 0.5
    # (a 16-dim block would give X = 2^-7 and 0.03125 instead)
    q[0, 0] = 0.75
    q[0, 20] = 0.0375
    # head 31, block 3: amax 1e-3 -> X = 2^-12 (byte 115); 4.096 -> 4
    q[31, 100] = -1e-3
    c, s = R.quant_indexer_q(q)
    assert c.shape == (32, 64) and s.shape == (32, 4)
    # codes: 5 -> 4 (6), -2.6 -> -3 (13), 0.3 -> 0.5 (1), 0.25 -> 0 (0),
    # 7 -> 6 (7), -0.1 -> -0 (8), 1.25 -> 1 (2); channel 2c in the low nibble
    assert list(c[3, 16:20]) == [0xD6, 0x01, 0x87, 0x02]
    assert s[3, 1] == 127 and s[0, 0] == 124 and s[31, 3] == 115
    assert s[0, 3] == 0 and np.all(c[0, 48:64] == 0)           # all-zero block
    d = R.dequant_mxfp4(c, s)
    assert list(d[3, 32:39]) == [4.0, -3.0, 0.5, 0.0, 6.0, 0.0, 1.0]
    assert d[0, 0] == 0.75 and d[0, 20] == 0.0625
    assert d[31, 100] == -4.0 * 2.0 ** -12
    # the score uses the quantised query: unit weight on head 3 against
    # unit keys e_32 and -e_33 gives relu(4) and relu(3)
    w = np.zeros(32); w[3] = 1.0
    k = np.zeros((3, 128)); k[0, 32] = 1.0; k[1, 33] = -1.0; k[2, 32] = -1.0
    assert list(R.index_scores_fp4q(q, w, k)) == [4.0, 3.0, 0.0]


def test_fp4q_exact_when_representable():
    """A query whose every (head, 32-dim block) is E2M1 values times its own
    power of two, with |max| 6 or 4, is its own MXFP4 form, so the scores
    equal the plain ones exactly.  The exponents differ by up to 2^40 from
    block to block, so a block taken along the wrong axis (across heads) or
    over 64 dims would crush the small blocks."""
    rng = np.random.default_rng(11)
    e2 = F.e2m1_value(np.arange(16))
    codes = rng.integers(0, 16, size=(32, 4, 32))
    codes[:, :, 0] = rng.choice([6, 7, 14, 15], size=(32, 4))      # |max| in {4, 6}
    ex = rng.integers(-20, 21, size=(32, 4))
    q = (e2[codes] * np.exp2(ex)[:, :, None]).reshape(32, 128)
    c, s = R.quant_indexer_q(q)
    assert np.array_equal(R.dequant_mxfp4(c, s), q)
    w = rng.uniform(0, 1, 32)
    k = rng.standard_normal((50, 128))
    assert np.array_equal(R.index_scores_fp4q(q, w, k), R.index_scores(q, w, k))


def test_fp4q_error_bound():
    """Each quantised element lies within 2 X of the input (amax / X is in
    [4, 8): half an E2M1 step is at most X below 6 X, saturation costs less
    than 2 X above it), and the relu is 1-Lipschitz, so
    |s_fp4 - s| <= sum_h w_h sum_c 2 X_hc |k_c|."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((32, 128)) * np.exp2(rng.integers(-6, 7, size=(32, 1)))
    w = rng.uniform(0, 1, 32)
    k = rng.standard_normal((64, 128))
    c, s = R.quant_indexer_q(q)
    X = np.repeat(F.e8m0_value(s), 32, axis=1)                   # [32, 128]
    qh = R.dequant_mxfp4(c, s)
    assert np.all(np.abs(qh - q) <= 2 * X)
    assert np.all(np.abs(qh - q) <= X * (np.abs(q) <= 6 * X) + 2 * X * (np.abs(q) > 6 * X))
    bound = (np.abs(k) @ (2 * X).T) @ w
    err = np.abs(R.index_scores_fp4q(q, w, k) - R.index_scores(q, w, k))
    assert np.all(err <= bound) and np.all(R.index_scores_fp4q(q, w, k) >= 0)
    # the quantisation is scale-equivariant under powers of two
    c2, s2 = R.quant_indexer_q(q * 2.0 ** 5)
    assert np.array_equal(c2, c) and np.array_equal(s2.astype(int), s.astype(int) + 5)


# ------------------------------------------------------------------ f2
def test_swa_row_worked_example():
    """FP8 SWA row: sigma = max|x| / 448 stored in fp32, codes
    RNE_E4M3FN(x / sigma) of the exact quotient."""
    x = np.zeros(512)
    x[:5] = [3.5, -1.75, 2.0 ** -7, 0.3, -0.0]
    c, sg = R.quant_swa_row(x)
    assert sg == np.float32(2.0 ** -7)                 # 3.5 / 448 = 2^-7 exactly
    # 3.5 / sigma = 448 -> 0x7E; -224 = -1.75 * 2^7 -> 0x80 | (14 << 3) | 6;
    # 1 -> 0x38; 0.3 / 2^-7 = 38.4 -> 40 (1.25 * 2^5: (12 << 3) | 2); -0 -> 0
    assert list(c[:5]) == [0x7E, 0xF6, 0x38, 0x62, 0x00]
    assert np.all(c[5:] == 0)
    z, zs = R.quant_swa_row(np.zeros(512))
    assert zs == 0 and np.all(z == 0)
    # sigma times the decoded code of the row maximum is the maximum itself
    rng = np.random.default_rng(21)
    rows = rng.standard_normal((20, 512)) * np.exp2(rng.integers(-20, 20, size=(20, 1)))
    c, sg = R.quant_swa_row(rows)
    dec = F.e4m3fn_value(c)
    top = np.abs(rows).argmax(axis=1)
    assert np.all(np.abs(dec[np.arange(20), top]) == 448.0)


def test_swa_row_nearest_brute_force():
    """Every code is a nearest E4M3FN value of the exact quotient x / sigma,
    ties to the even code, with sigma the fp32 number nearest max|x| / 448
    (numpy's fp32 division of fp32 inputs is correctly rounded)."""
    rng = np.random.default_rng(22)
    rows = rng.standard_normal((8, 512)).astype(np.float32)
    c, sg = R.quant_swa_row(rows)
    allc = np.arange(256)
    allv = F.e4m3fn_value(allc)
    fin = ~np.isnan(allv)
    for r in range(8):
        assert sg[r] == np.abs(rows[r]).max() / np.float32(448)
        v = rows[r].astype(np.float64) / np.float64(sg[r])
        d = np.abs(np.abs(v)[:, None] - np.abs(allv[None, fin]))
        best = d.min(axis=1)
        got = np.abs(np.abs(v) - np.abs(F.e4m3fn_value(c[r])))
        assert np.array_equal(got, best)
        assert np.all((c[r] >= 0x80) == (v < 0))


def test_swa_row_exact_quotient():
    """The code is taken from the exact quotient, not from a rounded one:
    with sigma = 2^-7 (a row maximum of 3.5) the element 2^-7 * (38 - 2^-20)
    lies just below the midpoint 38 of the E4M3 values 36 (code 0x61) and 40
    (code 0x62), so it rounds down to 36, although its quotient rounded to
    fp32 (a precision of 2^-18 there) would be exactly 38, which goes to the
    even code, 40."""
    x = np.zeros(512)
    x[0] = 3.5
    x[1] = 2.0 ** -7 * (38.0 - 2.0 ** -20)
    c, sg = R.quant_swa_row(x)
    assert sg == np.float32(2.0 ** -7)
    assert c[1] == 0x61
    assert np.float32(x[1] / 2.0 ** -7) == 38.0       # what an fp32 quotient would see
    x[1] = 2.0 ** -7 * 38.0                           # the midpoint itself: even code
    assert R.quant_swa_row(x)[0][1] == 0x62
    x[1] = 2.0 ** -7 * (38.0 + 2.0 ** -20)            # just above it
    assert R.quant_swa_row(x)[0][1] == 0x62


def test_append_matches_batch_build():
    """Appending T tokens one by one gives the entries that compressing the
    complete groups in one call gives (steps a1-a3 are pinned on their own),
    and leaves the incomplete group's tokens in the tail."""
    rng = np.random.default_rng(23)
    w_ik = rng.standard_normal((128, 512)) / 22.6
    for m in (1, 2, 4):
        T = 4 * m + (m - 1)
        h = rng.standard_normal((T, 512))
        z = rng.standard_normal((T, 512)) * 2
        sw = rng.standard_normal((T, 512))
        st = R.new_state(m, W=8)
        cache = dict(kv_codes=np.zeros((8, 256), np.uint8), kv_scales=np.zeros((8, 32), np.uint8),
                     ik_codes=np.zeros((8, 64), np.uint8), ik_scales=np.zeros((8, 4), np.uint8))
        for t in range(T):
            R.append_token(st, cache, h[t], z[t], sw[t], w_ik)
        n = T // m
        ref = R.build_entries(h[:n * m], None if m == 1 else z[:n * m], m, w_ik)
        for key in ("kv_codes", "kv_scales", "ik_codes", "ik_scales"):
            assert np.array_equal(cache[key][:n], ref[key]), (m, key)
            assert np.all(cache[key][n:] == 0)
        assert st["n_tok"] == T
        if m > 1:
            assert np.array_equal(st["tail_h"][:T - n * m], h[n * m:])
            assert np.array_equal(st["tail_z"][:T - n * m], z[n * m:])


def test_swa_ring_and_geometry():
    """Geometry of the next query and the ring window, before, at and past
    the wrap of a W = 8 ring; the window lists the last min(W, T) tokens'
    rows oldest first."""
    assert R.decode_geometry(0, 2, 8) == (0, 0, 0)
    assert R.decode_geometry(5, 2, 8) == (2, 0, 5)      # entries 0, 1 = tokens 0-3
    assert R.decode_geometry(8, 1, 8) == (8, 0, 8)
    assert R.decode_geometry(13, 4, 8) == (3, 5, 8)     # tokens 5..12 in slots 5,6,7,0..4
    rng = np.random.default_rng(24)
    w_ik = rng.standard_normal((128, 512)) / 22.6
    sw = rng.standard_normal((13, 512))
    st = R.new_state(1, W=8)
    cache = dict(kv_codes=np.zeros((16, 256), np.uint8), kv_scales=np.zeros((16, 32), np.uint8),
                 ik_codes=np.zeros((16, 64), np.uint8), ik_scales=np.zeros((16, 4), np.uint8))
    for t in range(13):
        R.append_token(st, cache, sw[t], None, sw[t], w_ik)
        _, start, ln = R.decode_geometry(t + 1, 1, 8)
        wc, ws = R.swa_window(st["swa_codes"], st["swa_scale"], start, ln)
        rc, rs = R.quant_swa_row(sw[t + 1 - ln:t + 1])
        assert np.array_equal(wc, rc) and np.array_equal(ws, rs)


# ------------------------------------------------------------------ f4
def test_rope_worked_example_and_identities():
    """RoPE on the last `dims` channels, adjacent pairs, angle pos *
    theta^(-2i/dims): values worked by hand for dims = 4, theta = 100."""
    x = np.zeros(512)
    x[508], x[510], x[100] = 1.0, 2.0, 7.0
    y = R.rope_rotate(x, np.pi / 2, 4, 100.0)
    # pair 0 (508, 509) turns by pi/2: (1, 0) -> (0, 1); pair 1 (510, 511) by
    # pi/20: (2, 0) -> (2 cos, 2 sin); channel 100 is not a RoPE channel
    assert abs(y[508]) < 1e-15 and y[509] == 1.0
    assert np.isclose(y[510], 2 * np.cos(np.pi / 20), rtol=1e-15)
    assert np.isclose(y[511], 2 * np.sin(np.pi / 20), rtol=1e-15)
    assert y[100] == 7.0 and np.count_nonzero(np.abs(y) > 1e-15) == 4
    rng = np.random.default_rng(31)
    v = rng.standard_normal((5, 512))
    assert np.array_equal(R.rope_rotate(v, 0, 64, 1e4), v)
    assert np.array_equal(R.rope_rotate(v, 123, 0, 1e4), v)
    a = R.rope_rotate(R.rope_rotate(v, 1000, 64, 1e4), 234567, 64, 1e4)
    assert np.allclose(a, R.rope_rotate(v, 235567, 64, 1e4), rtol=0, atol=1e-9)
    r = R.rope_rotate(v, 98765, 64, 1e4)
    assert np.array_equal(r[:, :448], v[:, :448])
    pn = lambda z: z[:, 448::2] ** 2 + z[:, 449::2] ** 2
    assert np.allclose(pn(r), pn(v), rtol=1e-12)
    # dot products depend only on the position difference
    q, k = rng.standard_normal(512), rng.standard_normal(512)
    d1 = R.rope_rotate(q, 500, 64, 1e4) @ R.rope_rotate(k, 530, 64, 1e4)
    d2 = R.rope_rotate(q, 70000, 64, 1e4) @ R.rope_rotate(k, 70030, 64, 1e4)
    assert np.isclose(d1, d2, rtol=1e-9)


def test_bf16_round():
    assert list(R.bf16_round([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20)])) == \
        [1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7)]        # ties to even, otherwise nearest
    x = np.random.default_rng(32).standard_normal(1000) * 100
    r = R.bf16_round(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(R.bf16_round(r), r)


def test_attend_rope_undoes_the_rows_rotation():
    """Rows that are a value set rotated by the query's own position give
    exactly the attention over the unrotated values (before the cast):
    dot products are rotation-invariant and the inverse RoPE undoes the
    rotation the mix carries.  A sign slip in either rotation breaks it."""
    rng = np.random.default_rng(33)
    q = rng.standard_normal((64, 512)) / np.sqrt(512)
    v = rng.standard_normal((40, 512))
    for pos in (0, 17, 1 << 20):
        rows = R.rope_rotate(v, pos, 64, 1e4)
        ob, o, lse = R.attend_rope(q, rows, pos, 64, 1e4)
        o_ref, lse_ref = R.attend(q, v)
        assert np.allclose(o, o_ref, rtol=0, atol=1e-11) and np.allclose(lse, lse_ref, atol=1e-11)
        assert np.array_equal(ob, R.bf16_round(o))
    # no RoPE channels: plain attention
    ob, o, lse = R.attend_rope(q, v, 5, 0, 1e4)
    assert np.array_equal(o, R.attend(q, v)[0])


# ------------------------------------------------------------------ a5
def test_topk_textbook_sort_with_ties():
    rng = np.random.default_rng(8)
    s = rng.integers(0, 6, 60).astype(float)          # many exact ties
    for k in (1, 5, 17, 60, 100):
        want = sorted(sorted(range(60), key=lambda j: (-s[j], j))[:k])
        assert list(R.topk(s, k)) == want
    # duplicates: the lowest index wins
    s = np.array([1.0, 3.0, 3.0, 3.0, 2.0])
    assert list(R.topk(s, 2)) == [1, 2]
    # explicit ids (a candidate pool)
    ids = np.array([10, 20, 30, 40, 50])
    assert list(R.topk(s, 2, ids)) == [20, 30]


def test_topk_subset_enumeration():
    # brute force: the selected set has the largest score sum among all
    # k-subsets, and the lowest index sum among those
    rng = np.random.default_rng(9)
    s = rng.integers(0, 4, 9).astype(float)
    k = 4
    best = max(itertools.combinations(range(9), k), key=lambda c: (sum(s[list(c)]), -sum(c)))
    assert list(R.topk(s, k)) == sorted(best)


# ------------------------------------------------------------------ a6
def test_block_pool_tiny_brute_force():
    s = np.array([0, 9, 1, 1, 5, 5, 5, 5, 2, 9, 0, 0, 7], dtype=float)
    # blocks of 4: maxima [9, 5, 9, 7] -> top 2 by (max desc, id asc) = blocks 0, 2
    assert list(R.block_pool(s, block=4, n_blocks=2)) == [0, 1, 2, 3, 8, 9, 10, 11]
    # top 3 adds block 3, which is partial (only position 12 visible)
    assert list(R.block_pool(s, block=4, n_blocks=3)) == [0, 1, 2, 3, 8, 9, 10, 11, 12]
    assert list(R.block_pool(s, block=4, n_blocks=10)) == list(range(13))


def test_block_pool_invariants():
    rng = np.random.default_rng(10)
    n = 40000
    s = rng.standard_normal(n) ** 2
    s[1000:1040] = s.max()                      # a run of exact ties
    pool = R.block_pool(s, 8, 2048)
    assert pool.size == 16384
    assert np.all(np.diff(pool) > 0)
    assert set(R.topk(s, 512)) <= set(pool)
    bm = R.block_max(s, 8)
    inpool = np.zeros(bm.size, bool); inpool[pool // 8] = True
    assert bm[inpool].min() >= bm[~inpool].max()
    # Reindex with the Full layer's own scores reproduces the Full top-512
    assert np.array_equal(R.topk(s[pool], 512, pool), R.topk(s, 512))


# ------------------------------------------------------------------ a9
def test_attend_special_cases():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((64, 512)) / math.sqrt(512)
    v = rng.standard_normal((1, 512))
    o, lse = R.attend(q, v)
    assert np.allclose(o, np.repeat(v, 64, 0), rtol=0, atol=1e-15)
    assert np.allclose(lse, q @ v[0], rtol=1e-14)
    v = rng.standard_normal((30, 512))
    o, lse = R.attend(np.zeros((64, 512)), v)
    assert np.allclose(o, np.repeat(v.mean(0, keepdims=True), 64, 0), atol=1e-14)
    assert np.allclose(lse, math.log(30))


def test_attend_library_softmax_and_permutation():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((64, 512)) / math.sqrt(512)
    v = rng.standard_normal((50, 512))
    o, lse = R.attend(q, v)
    p = scipy.special.softmax(q @ v.T, axis=1)
    assert np.allclose(o, p @ v, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, scipy.special.logsumexp(q @ v.T, axis=1), rtol=1e-13)
    perm = rng.permutation(50)
    o2, lse2 = R.attend(q, v[perm])
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-13)


def test_attend_split_merge():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((64, 512)) / math.sqrt(512)
    v = rng.standard_normal((100, 512)) * 3
    o, lse = R.attend(q, v)
    parts = [R.attend(q, v[a:b]) for a, b in ((0, 37), (37, 64), (64, 100))]
    L = np.stack([p[1] for p in parts])
    m = L.max(0)
    wts = np.exp(L - m)
    merged = sum(wts[i][:, None] * parts[i][0] for i in range(3)) / wts.sum(0)[:, None]
    assert np.allclose(merged, o, rtol=1e-12, atol=1e-13)
    assert np.allclose(m + np.log(wts.sum(0)), lse, rtol=1e-13)


def test_gather_rows_skips_padding_and_appends_swa():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((10, 512))
    c, s = R.quant_main_kv(x)
    swa_c = rng.integers(0, 0x7E, (3, 512)).astype(np.uint8)
    swa_s = np.array([0.5, 2.0, 0.25])
    rows = R.gather_rows(c, s, np.array([4, -1, 2]), swa_c, swa_s)
    assert rows.shape == (5, 512)
    assert np.array_equal(rows[0], R.dequant_main_kv(c[4], s[4]))
    assert np.array_equal(rows[3], F.e4m3fn_value(swa_c[1]) * 2.0)


# --------------------------------------------------- a1-a3 together
def test_build_entries_projects_the_stored_entry():
    """Hand-worked entry (tests/golden/xhat_projection_example.json): the
    indexer K is projected from the dequantised main KV, whose channel 1 is
    1.0 where the raw latent holds 0.9, and the two readings give different
    MXFP4 bytes."""
    import json
    import os
    G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "xhat_projection_example.json")))
    h = np.zeros((1, 512))
    for c, v in G["h_nonzero"].items():
        h[0, int(c)] = v
    w_ik = np.zeros((128, 512))
    for d, c, v in G["w_ik_nonzero"]:
        w_ik[d, c] = v
    e = R.build_entries(h, None, 1, w_ik)
    assert e["kv_codes"][0, 0] == G["kv_codes_byte0"] and np.all(e["kv_codes"][0, 1:] == 0)
    assert e["kv_scales"][0, 0] == G["kv_scales_byte0"] and np.all(e["kv_scales"][0, 1:] == 0)
    want_ik = np.zeros(64, np.uint8)
    for b, v in G["ik_codes"].items():
        want_ik[int(b)] = v
    assert np.array_equal(e["ik_codes"][0], want_ik)
    assert e["ik_scales"][0].tolist() == G["ik_scales"]
    khat = R.dequant_mxfp4(e["ik_codes"], e["ik_scales"])
    assert khat[0, 0] == G["khat0"] and np.all(khat[0, 1:] == 0)
    assert khat[0, 0] != G["khat0_if_x_were_projected"]


def test_kth_score_by_hand():
    """The k-th best score of small lists worked by hand: ties count once per
    candidate, and k beyond the list gives its smallest score."""
    s = [3.0, 1.0, 4.0, 1.0, 5.0, 9.0, 2.0, 6.0]
    assert R.kth_score(s, 1) == 9.0
    assert R.kth_score(s, 3) == 5.0            # 9, 6, 5
    assert R.kth_score(s, 7) == 1.0            # 9 6 5 4 3 2 1
    assert R.kth_score(s, 100) == 1.0
    assert R.kth_score([2.0, 2.0, 2.0, 1.0], 2) == 2.0
    assert R.kth_score([2.0, 2.0, 2.0, 1.0], 4) == 1.0
    assert R.kth_score([-1.0, 0.5, -3.0], 2) == -1.0
