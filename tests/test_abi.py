"""The C-ABI library loads, exports every function include/csa2.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_csa2_amd as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: every call below fails validation


def declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol():
    L = C.lib()
    names = declared()
    assert set(names) == set(C.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_constants_match_the_header():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    for name in ("CSA2_MAX_K", "CSA2_MAX_COLS", "CSA2_OP_TOPK", "CSA2_OP_POOL", "CSA2_OP_ATTEND",
                 "CSA2_OP_SELECT_ATTEND", "CSA2_OP_POOL_ATTEND"):
        m = re.search(r"#define\s+" + name + r"\s+(\(1 << \d+\)|\d+)", src)
        assert m, name
        assert eval(m.group(1)) == getattr(C, name), name


def test_status_strings():
    L = C.lib()
    assert L.csa2_status_string(0) == b"CSA2_OK"
    assert L.csa2_status_string(4) == b"CSA2_EHIP"
    assert L.csa2_status_string(99) == b"CSA2_UNKNOWN"


def _cache(cap=100, ptr=0x10000, batch=0):
    return C._Cache(ptr, ptr, ptr, ptr, cap, batch)


def test_compress_validation():
    L = C.lib()
    cs = _cache(cap=100)
    # null h
    assert L.csa2_compress_quant(None, None, 1, 64, 1, FAKE, ctypes.byref(cs), 0, None) == 1
    # T not a multiple of m
    assert L.csa2_compress_quant(FAKE, FAKE, 1, 63, 2, FAKE, ctypes.byref(cs), 0, None) == 1
    assert b"multiple" in L.csa2_last_error()
    # m > 1 without logits
    assert L.csa2_compress_quant(FAKE, None, 1, 64, 2, FAKE, ctypes.byref(cs), 0, None) == 1
    # past the cache capacity
    assert L.csa2_compress_quant(FAKE, None, 1, 101, 1, FAKE, ctypes.byref(cs), 0, None) == 1
    assert L.csa2_compress_quant(FAKE, None, 1, 60, 1, FAKE, ctypes.byref(cs), 41, None) == 1
    # misaligned cache array
    bad = _cache(ptr=0x10004)
    assert L.csa2_compress_quant(FAKE, None, 1, 8, 1, FAKE, ctypes.byref(bad), 0, None) == 1
    assert b"aligned" in L.csa2_last_error()
    # m out of range
    assert L.csa2_compress_quant(FAKE, FAKE, 1, 34, 17, FAKE, ctypes.byref(cs), 0, None) == 1
    # a negative batch count in the cache struct
    neg = _cache(batch=-1)
    assert L.csa2_compress_quant(FAKE, None, 1, 8, 1, FAKE, ctypes.byref(neg), 0, None) == 1
    assert b"batch" in L.csa2_last_error()


@pytest.mark.parametrize("entry", ["csa2_index_score", "csa2_index_score_fp4q"])
def test_index_score_validation(entry):
    L = C.lib()
    cs = _cache(cap=100)
    P = FAKE
    f = getattr(L, entry)
    assert f(None, P, P, P, None, 0, 1, 10, ctypes.byref(cs), P, 10, None) == 1
    assert f(P, P, P, P, None, 0, 0, 10, ctypes.byref(cs), P, 10, None) == 1
    assert f(P, P, P, P, None, 0, 1, 10, ctypes.byref(cs), P, 9, None) == 1
    assert f(P, P, P, P, None, 0, 1, 101, ctypes.byref(cs), P, 101, None) == 1
    assert f(P, P, P, P, P, 5, 1, 10, ctypes.byref(cs), P, 10, None) == 1
    # a score row of 2^29 columns or more (the row is addressed in 32-bit bytes)
    big = _cache(cap=1 << 30)
    assert f(P, P, P, P, None, 0, 1, 1 << 29, ctypes.byref(big), P, 1 << 29, None) == 1
    assert b"2^29" in L.csa2_last_error()
    # nothing to score: returns OK without launching
    assert f(P, P, P, P, None, 0, 1, 0, ctypes.byref(cs), P, 10, None) == 0


def test_select_and_pool_validation():
    L = C.lib()
    P = FAKE
    for k in (0, -1, 2049):
        assert L.csa2_select_topk(P, 100, 1, P, None, 100, k, P, None, 0, None) == 1
    assert L.csa2_select_topk(P, 100, 1, P, None, 101, 5, P, None, 0, None) == 1
    assert L.csa2_select_topk(P, 1 << 25, 1, P, None, (1 << 24) + 1, 5, P, None, 0, None) == 1
    # workspace needed above 16384 columns
    assert L.csa2_select_topk(P, 20000, 1, P, None, 20000, 5, P, None, 0, None) == 3
    need = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, 1, 20000, 5)
    assert need == 4 * 2512                 # 2500 block maxima, rows padded to 16 words
    assert L.csa2_select_topk(P, 20000, 1, P, None, 20000, 5, P, P, need - 1, None) == 3
    assert L.csa2_block_pool(P, 100, 1, P, 100, 16, 4, P, P, 0, None, P, 1 << 20, None) == 2
    assert L.csa2_block_pool(P, 100, 1, P, 100, 8, 0, P, P, 0, None, P, 1 << 20, None) == 1
    assert L.csa2_block_pool(P, 100, 1, P, 100, 8, 4, None, P, 0, None, P, 1 << 20, None) == 1
    # fused top-k: k above the block count, or no output buffer
    assert L.csa2_block_pool(P, 100, 1, P, 100, 8, 4, P, P, 5, P, P, 1 << 20, None) == 1
    assert L.csa2_block_pool(P, 100, 1, P, 100, 8, 4, P, P, 3, None, P, 1 << 20, None) == 1


def test_select_noalloc_validation():
    """The allocation-free top-k validates like csa2_select_topk and refuses,
    before any HIP call, a size whose maxima exceed its static scratch."""
    L = C.lib()
    P = FAKE
    assert L.csa2_select_topk_noalloc(P, 100, 1, P, None, 100, 5, None, None) == 1
    assert L.csa2_select_topk_noalloc(P, 100, 1, P, None, 100, 0, P, None) == 1
    assert L.csa2_select_topk_noalloc(P, 100, 1, P, None, 101, 5, P, None) == 1
    Q, n = 64, 1 << 19
    assert C.csa2_workspace_bytes(C.CSA2_OP_TOPK, Q, n, 512) > 16 << 20
    assert L.csa2_select_topk_noalloc(P, n, Q, P, None, n, 512, P, None) == 2
    assert b"static" in L.csa2_last_error()


def test_attend_validation():
    L = C.lib()
    cs = _cache()
    P = FAKE
    assert L.csa2_sparse_attend(None, P, 1, ctypes.byref(cs), P, 8, P, P, 4, P, P, P, None, None, 0, None) == 1
    assert L.csa2_sparse_attend(P, P, 1, ctypes.byref(cs), None, 8, P, P, 4, P, P, P, None, None, 0, None) == 1
    assert L.csa2_sparse_attend(P, P, 1, ctypes.byref(cs), P, 4096, P, P, 4, P, P, P, None, None, 0, None) == 1
    assert L.csa2_sparse_attend(P, P, 1, ctypes.byref(cs), P, 8, None, None, 4, P, P, P, None, None, 0, None) == 1
    assert L.csa2_sparse_attend(P, P, 0, ctypes.byref(cs), P, 8, P, P, 4, P, P, P, None, None, 0, None) == 1
    assert L.csa2_sparse_attend(P, P, 1, None, P, 8, P, P, 4, P, P, P, None, None, 0, None) == 1


def test_attend_rope_validation():
    L = C.lib()
    cs = _cache()
    P = FAKE

    def call(rope, out=P):
        r = None if rope is None else ctypes.byref(rope)
        return L.csa2_sparse_attend_rope(P, P, 1, ctypes.byref(cs), P, 8, P, P, 4, P, P, r, out,
                                         None, None, 0, None)

    assert call(None) == 1
    assert call(C._Rope(0x10000, 64, 1e4), out=None) == 1
    assert call(C._Rope(0x10000, 63, 1e4)) == 1              # odd
    assert call(C._Rope(0x10000, 66, 1e4)) == 1              # past the last 64 channels
    assert call(C._Rope(0x10000, -2, 1e4)) == 1
    assert call(C._Rope(None, 64, 1e4)) == 1                 # positions needed
    assert call(C._Rope(0x10000, 64, 1.0)) == 1              # base must exceed 1
    assert call(C._Rope(0x10000, 64, float("inf"))) == 1
    assert call(C._Rope(0x10004, 64, 1e4)) == 1              # misaligned positions
    assert b"q_pos" in L.csa2_last_error()


def test_decode_append_validation():
    L = C.lib()
    cs = _cache()
    P = FAKE
    ok = dict(tail_h=0x10000, tail_z=0x10000, n_tok=0x10000, swa_codes=0x10000, swa_scale=0x10000)

    def state(**kw):
        d = dict(ok, W=8, m=2)
        d.update(kw)
        return C._State(d["tail_h"], d["tail_z"], d["n_tok"], d["swa_codes"], d["swa_scale"],
                        d["W"], d["m"])

    def call(h=P, z=P, sw=P, B=2, w=P, cache=cs, st=None):
        st = state() if st is None else st
        return L.csa2_decode_append(h, z, sw, B, w, ctypes.byref(cache), ctypes.byref(st),
                                    None, None, None, None)

    assert call(h=None) == 1
    assert call(w=None) == 1
    assert call(B=0) == 1 and call(B=65536) == 1
    assert call(st=state(m=0)) == 1 and call(st=state(m=17)) == 1
    assert call(st=state(W=129)) == 1 and call(st=state(W=-1)) == 1
    assert call(st=state(n_tok=0)) == 1
    assert call(z=None) == 1                                  # m = 2 needs the logits
    assert call(st=state(tail_h=0)) == 1
    assert call(sw=None) == 1                                 # W > 0 needs the SWA latent
    assert call(st=state(swa_codes=0)) == 1
    assert call(h=ctypes.c_void_p(0x10008)) == 1              # misaligned
    assert b"aligned" in L.csa2_last_error()
    assert call(cache=_cache(ptr=0x10004)) == 1


def test_workspace_sizes():
    # top-k / pool: the 8-way maxima levels up to the first one with <= 16384 groups
    n = 1 << 20
    assert C.csa2_workspace_bytes(C.CSA2_OP_TOPK, 4, n, 512) == 4 * 4 * (n // 8 + n // 64)
    assert C.csa2_workspace_bytes(C.CSA2_OP_TOPK, 4, 16384, 512) == 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_POOL, 4, 16384, 2048) == 4 * 4 * 2048
    # attention: partial (max, sum, O) per split for small batches, none for large
    assert C.csa2_workspace_bytes(C.CSA2_OP_ATTEND, 4, 0, 512) > 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_ATTEND, 4096, 0, 512) == 0


def test_selftest_counter_query():
    assert C.lib().csa2_selftest(None, 0, None) == 9


def test_alignment_validation():
    """Every array must be aligned to at least its element size: a pointer
    off by 4 bytes for an int64 array, or by 2 bytes for an int32 / fp32 one,
    is refused on the host with CSA2_EINVAL.  Each call below is otherwise
    one that stops before any launch (a short workspace, nothing to score,
    an empty batch), so a missing check shows as a status other than EINVAL."""
    L = C.lib()
    P = FAKE
    A4 = ctypes.c_void_p(0x10004)        # 4-byte aligned, not 8
    A2 = ctypes.c_void_p(0x10002)        # 2-byte aligned, not 4
    cs = _cache(cap=1 << 20)

    def einval(st):
        assert st == 1, st
        assert b"aligned" in L.csa2_last_error(), L.csa2_last_error()

    # index scores (n_cols = 0: returns before any launch once validated)
    for entry in ("csa2_index_score", "csa2_index_score_fp4q"):
        f = getattr(L, entry)
        assert f(P, P, P, P, None, 0, 1, 0, ctypes.byref(cs), P, 10, None) == 0
        einval(f(P, P, A2, P, None, 0, 1, 0, ctypes.byref(cs), P, 10, None))    # q_seq
        einval(f(P, P, P, A4, None, 0, 1, 0, ctypes.byref(cs), P, 10, None))    # n_vis
        einval(f(P, P, P, P, A2, 10, 1, 0, ctypes.byref(cs), P, 10, None))      # cand
        einval(f(P, A2, P, P, None, 0, 1, 0, ctypes.byref(cs), P, 10, None))    # w
        einval(f(P, P, P, P, None, 0, 1, 0, ctypes.byref(cs), A2, 10, None))    # scores
    # top-k (20000 columns with no workspace: CSA2_EWORKSPACE once validated)
    n = 20000
    assert L.csa2_select_topk(P, n, 1, P, None, n, 5, P, None, 0, None) == 3
    einval(L.csa2_select_topk(P, n, 1, P, None, n, 5, A2, None, 0, None))       # out
    einval(L.csa2_select_topk(P, n, 1, A4, None, n, 5, P, None, 0, None))       # n_valid
    einval(L.csa2_select_topk(P, n, 1, P, A2, n, 5, P, None, 0, None))          # col_ids
    einval(L.csa2_select_topk(A2, n, 1, P, None, n, 5, P, None, 0, None))       # scores
    assert L.csa2_select_topk_levels(P, n, 1, P, None, n, 5, P, None, 0, None) == 3
    einval(L.csa2_select_topk_levels(P, n, 1, P, None, n, 5, A2, None, 0, None))
    einval(L.csa2_select_topk_levels(P, n, 1, A4, None, n, 5, P, None, 0, None))
    # the allocation-free top-k (a size past its static scratch: EUNSUPPORTED)
    Q, m = 64, 1 << 19
    assert L.csa2_select_topk_noalloc(P, m, Q, P, None, m, 512, P, None) == 2
    einval(L.csa2_select_topk_noalloc(P, m, Q, P, None, m, 512, A2, None))
    einval(L.csa2_select_topk_noalloc(P, m, Q, A4, None, m, 512, P, None))
    einval(L.csa2_select_topk_noalloc(P, m, Q, P, A2, m, 512, P, None))
    # block pool with its top-k
    assert L.csa2_block_pool(P, n, 1, P, n, 8, 4, P, P, 4, P, None, 0, None) == 3
    einval(L.csa2_block_pool(P, n, 1, P, n, 8, 4, A2, P, 4, P, None, 0, None))  # pool
    einval(L.csa2_block_pool(P, n, 1, P, n, 8, 4, P, A4, 4, P, None, 0, None))  # pool_len
    einval(L.csa2_block_pool(P, n, 1, P, n, 8, 4, P, P, 4, A2, None, 0, None))  # topk
    einval(L.csa2_block_pool(P, n, 1, A4, n, 8, 4, P, P, 4, P, None, 0, None))  # n_valid

    # fused selection + attention (no workspace: CSA2_EWORKSPACE once validated)
    def sa(entry="csa2_select_attend", **kw):
        a = dict(scores=P, n_valid=P, col_ids=None, idx=P, pool=P, pool_len=P, q=P, q_seq=P,
                 swa_codes=P, swa_scale=P, swa_start=P, swa_len=P, out=P, lse=P)
        a.update(kw)
        return getattr(L, entry)(a["scores"], n, 1, a["n_valid"], a["col_ids"], n, 4, a["idx"], 4,
                                 a["pool"], a["pool_len"], a["q"], a["q_seq"], ctypes.byref(cs),
                                 a["swa_codes"], a["swa_scale"], 8, a["swa_start"], a["swa_len"],
                                 a["out"], a["lse"], None, 0, None)

    assert sa() == 3 and sa("csa2_select_attend_levels") == 3
    for name, bad in (("n_valid", A4), ("idx", A2), ("pool", A2), ("pool_len", A4),
                      ("q_seq", A2), ("swa_scale", A2), ("swa_start", A4), ("swa_len", A2),
                      ("lse", A2), ("scores", A2), ("out", ctypes.c_void_p(0x10008)),
                      ("q", ctypes.c_void_p(0x10008))):
        einval(sa(**{name: bad}))
        einval(sa("csa2_select_attend_levels", **{name: bad}))
    assert sa(pool=ctypes.c_void_p(0x10004)) == 3    # the pool needs only 4-byte alignment

    # attention (Q = 0: refused after the alignment checks, for another reason)
    def at(**kw):
        a = dict(q=P, q_seq=P, idx=P, swa_codes=P, swa_scale=P, swa_start=P, swa_len=P, out=P,
                 lse=P)
        a.update(kw)
        return L.csa2_sparse_attend(a["q"], a["q_seq"], 0, ctypes.byref(cs), a["idx"], 8,
                                    a["swa_codes"], a["swa_scale"], 4, a["swa_start"],
                                    a["swa_len"], a["out"], a["lse"], None, 0, None)

    assert at() == 1 and b"aligned" not in L.csa2_last_error()
    for name, bad in (("q_seq", A2), ("idx", A2), ("swa_scale", A2), ("swa_start", A4),
                      ("swa_len", A2), ("lse", A2), ("out", ctypes.c_void_p(0x10008))):
        einval(at(**{name: bad}))


def test_decode_append_output_alignment():
    L = C.lib()
    cs = _cache()
    P = FAKE
    st = C._State(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 8, 2)
    for nv, ss, sl in ((0x10004, None, None), (None, 0x10004, None), (None, None, 0x10002)):
        r = L.csa2_decode_append(P, P, P, 2, P, ctypes.byref(cs), ctypes.byref(st),
                                 None if nv is None else ctypes.c_void_p(nv),
                                 None if ss is None else ctypes.c_void_p(ss),
                                 None if sl is None else ctypes.c_void_p(sl), None)
        assert r == 1 and b"aligned" in L.csa2_last_error()
