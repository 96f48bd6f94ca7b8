"""Python binding of libcsa2, the MI355X (gfx950) CSA2 global-attention path.

Every function here only marshals arguments (torch tensors -> device
pointers, the current HIP stream) and calls the C ABI of the same name in
include/csa2.h; all computation runs in the library's HIP kernels.  PyTorch
supplies device memory and streams.  If libcsa2.so is missing the functions
raise: there is no CPU fallback.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIB selects another build of the library (the sanitizer build of the
# host code that a CPU test loads); by default the in-tree libcsa2.so.
LIB_PATH = os.environ.get("CSA2_LIB") or os.path.join(_PKG, "libcsa2.so")

CSA2_OP_TOPK, CSA2_OP_POOL, CSA2_OP_ATTEND = 1, 2, 3
CSA2_OP_SELECT_ATTEND, CSA2_OP_POOL_ATTEND = 4, 5
CSA2_MAX_K, CSA2_MAX_COLS = 2048, 1 << 24          # as include/csa2.h
STATUS = {0: "CSA2_OK", 1: "CSA2_EINVAL", 2: "CSA2_EUNSUPPORTED", 3: "CSA2_EWORKSPACE", 4: "CSA2_EHIP"}
EXPORTS = ("csa2_status_string", "csa2_last_error", "csa2_compress_quant", "csa2_index_score",
           "csa2_index_score_fp4q", "csa2_select_topk", "csa2_block_pool", "csa2_sparse_attend",
           "csa2_sparse_attend_rope", "csa2_decode_append", "csa2_workspace_bytes",
           "csa2_selftest", "csa2_select_topk_noalloc", "csa2_select_attend",
           "csa2_index_score_levels", "csa2_select_attend_levels", "csa2_select_topk_levels",
           "csa2_peak_read", "csa2_peak_mfma")


class Csa2Error(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [("kv_codes", ctypes.c_void_p), ("kv_scales", ctypes.c_void_p),
                ("ik_codes", ctypes.c_void_p), ("ik_scales", ctypes.c_void_p),
                ("cap", ctypes.c_int64), ("batch", ctypes.c_int64)]


class _Rope(ctypes.Structure):
    _fields_ = [("q_pos", ctypes.c_void_p), ("dims", ctypes.c_int), ("theta", ctypes.c_float)]


class _State(ctypes.Structure):
    _fields_ = [("tail_h", ctypes.c_void_p), ("tail_z", ctypes.c_void_p),
                ("n_tok", ctypes.c_void_p), ("swa_codes", ctypes.c_void_p),
                ("swa_scale", ctypes.c_void_p), ("W", ctypes.c_int64), ("m", ctypes.c_int)]


_lib = None


def lib():
    """Load libcsa2.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_status_string.argtypes = [I]
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_last_error.argtypes = []
        L.csa2_compress_quant.restype = I
        L.csa2_compress_quant.argtypes = [P, P, I, I64, I, P, ctypes.POINTER(_Cache), I64, P]
        for fn in (L.csa2_index_score, L.csa2_index_score_fp4q):
            fn.restype = I
            fn.argtypes = [P, P, P, P, P, I64, I, I64, ctypes.POINTER(_Cache), P, I64, P]
        for fn in (L.csa2_select_topk, L.csa2_select_topk_levels):
            fn.restype = I
            fn.argtypes = [P, I64, I, P, P, I64, I, P, P, SZ, P]
        for fn in (L.csa2_select_attend, L.csa2_select_attend_levels):
            fn.restype = I
            fn.argtypes = [P, I64, I, P, P, I64, I, P, I, P, P, P, P,
                           ctypes.POINTER(_Cache), P, P, I64, P, P, P, P, P, SZ, P]
        L.csa2_index_score_levels.restype = I
        L.csa2_index_score_levels.argtypes = [P, P, P, P, I, I64, ctypes.POINTER(_Cache), P, I64,
                                              I, I, P, SZ, P]
        L.csa2_select_topk_noalloc.restype = I
        L.csa2_select_topk_noalloc.argtypes = [P, I64, I, P, P, I64, I, P, P]
        L.csa2_block_pool.restype = I
        L.csa2_block_pool.argtypes = [P, I64, I, P, I64, I, I, P, P, I, P, P, SZ, P]
        L.csa2_sparse_attend.restype = I
        L.csa2_sparse_attend.argtypes = [P, P, I, ctypes.POINTER(_Cache), P, I, P, P, I64, P, P,
                                         P, P, P, SZ, P]
        L.csa2_sparse_attend_rope.restype = I
        L.csa2_sparse_attend_rope.argtypes = [P, P, I, ctypes.POINTER(_Cache), P, I, P, P, I64, P,
                                              P, ctypes.POINTER(_Rope), P, P, P, SZ, P]
        L.csa2_decode_append.restype = I
        L.csa2_decode_append.argtypes = [P, P, P, I, P, ctypes.POINTER(_Cache),
                                         ctypes.POINTER(_State), P, P, P, P]
        L.csa2_workspace_bytes.restype = SZ
        L.csa2_workspace_bytes.argtypes = [I, I, I64, I]
        L.csa2_peak_read.restype = I
        L.csa2_peak_read.argtypes = [P, SZ, P, P]
        L.csa2_peak_mfma.restype = ctypes.c_double
        L.csa2_peak_mfma.argtypes = [I, P, P]
        L.csa2_selftest.restype = I
        L.csa2_selftest.argtypes = [P, I, P]
        _lib = L
    return _lib


# ------------------------------------------------------------ helpers
def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if ref is not None and ref.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(ref.device).cuda_stream)
    return ctypes.c_void_p(0)


def _check(fn, st):
    if st != 0:
        raise Csa2Error(fn, st, lib().csa2_last_error().decode())


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError(f"{name} must be {dt}, got {t.dtype}")


class Cache:
    """One KV-producing layer's global KV for B sequences: four device arrays
    (structure of arrays, 356 bytes per entry) allocated by torch."""

    def __init__(self, B, cap, device):
        self.B, self.cap = B, cap
        self.kv_codes = torch.empty(B, cap, 256, dtype=torch.uint8, device=device)
        self.kv_scales = torch.empty(B, cap, 32, dtype=torch.uint8, device=device)
        self.ik_codes = torch.empty(B, cap, 64, dtype=torch.uint8, device=device)
        self.ik_scales = torch.empty(B, cap, 4, dtype=torch.uint8, device=device)

    def c_struct(self):
        return _Cache(self.kv_codes.data_ptr(), self.kv_scales.data_ptr(),
                      self.ik_codes.data_ptr(), self.ik_scales.data_ptr(), self.cap, self.B)

    def view(self, b0, b1):
        """The same cache restricted to sequences b0..b1-1 (no copy)."""
        v = Cache.__new__(Cache)
        v.B, v.cap = b1 - b0, self.cap
        for name, arr in self.arrays().items():
            setattr(v, name, arr[b0:b1])
        return v

    def arrays(self):
        return dict(kv_codes=self.kv_codes, kv_scales=self.kv_scales,
                    ik_codes=self.ik_codes, ik_scales=self.ik_scales)

    @property
    def nbytes(self):
        return sum(a.numel() for a in self.arrays().values())


class State:
    """One KV-producing layer's decode state for B sequences (allocated by
    torch, zeroed: n_tok = 0): the tail of the incomplete group of m tokens
    and the SWA ring of W rows."""

    def __init__(self, B, m, W, device):
        self.B, self.m, self.W = B, m, W
        t = max(m - 1, 1)
        self.tail_h = torch.zeros(B, t, 512, dtype=torch.bfloat16, device=device)
        self.tail_z = torch.zeros(B, t, 512, dtype=torch.bfloat16, device=device)
        self.n_tok = torch.zeros(B, dtype=torch.int64, device=device)
        self.swa_codes = torch.zeros(B, max(W, 1), 512, dtype=torch.uint8, device=device)
        self.swa_scale = torch.zeros(B, max(W, 1), dtype=torch.float32, device=device)

    def view(self, b0, b1):
        """The same state restricted to sequences b0..b1-1 (no copy)."""
        v = State.__new__(State)
        v.B, v.m, v.W = b1 - b0, self.m, self.W
        for name in ("tail_h", "tail_z", "n_tok", "swa_codes", "swa_scale"):
            setattr(v, name, getattr(self, name)[b0:b1])
        return v

    def c_struct(self):
        return _State(self.tail_h.data_ptr(), self.tail_z.data_ptr(), self.n_tok.data_ptr(),
                      self.swa_codes.data_ptr(), self.swa_scale.data_ptr(), self.W, self.m)


# ------------------------------------------------------------ entry points
def csa2_workspace_bytes(op, Q, n_cols, k):
    return int(lib().csa2_workspace_bytes(op, Q, n_cols, k))


def csa2_compress_quant(h, z, m, w_ik, cache, e0=0, stream=None):
    """h, z: [B, T, 512] bf16 (z None iff m == 1); w_ik [128, 512] bf16."""
    _dtype(h, torch.bfloat16, "h"); _dtype(z, torch.bfloat16, "z"); _dtype(w_ik, torch.bfloat16, "w_ik")
    B, T = h.shape[0], h.shape[1]
    cs = cache.c_struct()
    st = lib().csa2_compress_quant(_ptr(h), _ptr(z), B, T, m, _ptr(w_ik), ctypes.byref(cs), e0,
                                   _stream(stream, h))
    _check("csa2_compress_quant", st)


def csa2_index_score(q_idx, w, q_seq, n_vis, cand, n_cols, cache, scores, stream=None,
                     fp4q=False):
    """q_idx [Q, 32, 128] bf16, w [Q, 32] f32, q_seq [Q] i32, n_vis [Q] i64,
    cand None or [Q, P] i32, scores [Q, ld] f32.  fp4q=True calls
    csa2_index_score_fp4q (the query quantised to MXFP4 first)."""
    _dtype(q_idx, torch.bfloat16, "q_idx"); _dtype(w, torch.float32, "w")
    _dtype(q_seq, torch.int32, "q_seq"); _dtype(n_vis, torch.int64, "n_vis")
    _dtype(cand, torch.int32, "cand"); _dtype(scores, torch.float32, "scores")
    Q = q_idx.shape[0]
    ld_cand = cand.shape[1] if cand is not None else 0
    cs = cache.c_struct()
    name = "csa2_index_score_fp4q" if fp4q else "csa2_index_score"
    st = getattr(lib(), name)(_ptr(q_idx), _ptr(w), _ptr(q_seq), _ptr(n_vis), _ptr(cand),
                              ld_cand, Q, n_cols, ctypes.byref(cs), _ptr(scores),
                              scores.shape[1], _stream(stream, q_idx))
    _check(name, st)


def csa2_index_score_levels(q_idx, w, q_seq, n_vis, n_cols, cache, scores, ws, n_blocks=0,
                            fp4q=False, stream=None):
    """csa2_index_score over all columns (no candidate list) that also writes
    the selection's maxima levels into ws (the workspace of the
    csa2_select_attend(..., levels=True) call that follows, of the same
    n_blocks sign)."""
    _dtype(q_idx, torch.bfloat16, "q_idx"); _dtype(w, torch.float32, "w")
    _dtype(q_seq, torch.int32, "q_seq"); _dtype(n_vis, torch.int64, "n_vis")
    _dtype(scores, torch.float32, "scores")
    Q = q_idx.shape[0]
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    cs = cache.c_struct()
    st = lib().csa2_index_score_levels(_ptr(q_idx), _ptr(w), _ptr(q_seq), _ptr(n_vis), Q, n_cols,
                                       ctypes.byref(cs), _ptr(scores), scores.shape[1], int(fp4q),
                                       n_blocks, _ptr(ws), wsb, _stream(stream, q_idx))
    _check("csa2_index_score_levels", st)


def csa2_select_topk(scores, n_valid, col_ids, n_cols, k, out, ws=None, stream=None,
                     levels=False):
    """scores [Q, ld] f32, n_valid [Q] i64, col_ids None or [Q, ld] i32,
    out [Q, k] i32; ws a uint8 tensor of csa2_workspace_bytes(TOPK, ...).
    levels=True calls csa2_select_topk_levels: ws already holds the maxima
    levels that csa2_index_score_levels (n_blocks=0) wrote for these scores."""
    _dtype(scores, torch.float32, "scores"); _dtype(n_valid, torch.int64, "n_valid")
    _dtype(col_ids, torch.int32, "col_ids"); _dtype(out, torch.int32, "out")
    Q = scores.shape[0]
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    name = "csa2_select_topk_levels" if levels else "csa2_select_topk"
    st = getattr(lib(), name)(_ptr(scores), scores.shape[1], Q, _ptr(n_valid), _ptr(col_ids),
                              n_cols, k, _ptr(out), _ptr(ws), wsb, _stream(stream, scores))
    _check(name, st)


def csa2_select_topk_noalloc(scores, n_valid, col_ids, n_cols, k, out, stream=None):
    """csa2_select_topk without a workspace (the library's static scratch)."""
    _dtype(scores, torch.float32, "scores"); _dtype(n_valid, torch.int64, "n_valid")
    _dtype(col_ids, torch.int32, "col_ids"); _dtype(out, torch.int32, "out")
    Q = scores.shape[0]
    st = lib().csa2_select_topk_noalloc(_ptr(scores), scores.shape[1], Q, _ptr(n_valid),
                                        _ptr(col_ids), n_cols, k, _ptr(out), _stream(stream, scores))
    _check("csa2_select_topk_noalloc", st)


def csa2_select_attend(scores, n_valid, col_ids, n_cols, k, idx, q, q_seq, cache, swa_codes,
                       swa_scale, swa_start, swa_len, out, lse=None, ws=None, n_blocks=0,
                       pool=None, pool_len=None, stream=None, levels=False):
    """Top-k (n_blocks == 0, col_ids optional) or pool + top-k (n_blocks > 0)
    fused with the attention over the selected rows; idx [Q, k] i32, out
    [Q, 64, 512] f32; ws from workspace(CSA2_OP_SELECT_ATTEND or
    CSA2_OP_POOL_ATTEND, Q, n_cols, k).  levels=True calls
    csa2_select_attend_levels: ws already holds the maxima levels that
    csa2_index_score_levels wrote for these scores."""
    _dtype(scores, torch.float32, "scores"); _dtype(n_valid, torch.int64, "n_valid")
    _dtype(col_ids, torch.int32, "col_ids"); _dtype(idx, torch.int32, "idx")
    _dtype(pool, torch.int32, "pool"); _dtype(pool_len, torch.int64, "pool_len")
    _dtype(q, torch.bfloat16, "q"); _dtype(q_seq, torch.int32, "q_seq")
    _dtype(swa_codes, torch.uint8, "swa_codes"); _dtype(swa_scale, torch.float32, "swa_scale")
    _dtype(swa_start, torch.int64, "swa_start"); _dtype(swa_len, torch.int32, "swa_len")
    _dtype(out, torch.float32, "out"); _dtype(lse, torch.float32, "lse")
    Q = scores.shape[0]
    T_swa = swa_codes.shape[1] if swa_codes is not None else 0
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    cs = cache.c_struct()
    name = "csa2_select_attend_levels" if levels else "csa2_select_attend"
    st = getattr(lib(), name)(_ptr(scores), scores.shape[1], Q, _ptr(n_valid), _ptr(col_ids),
                              n_cols, k, _ptr(idx), n_blocks, _ptr(pool), _ptr(pool_len),
                              _ptr(q), _ptr(q_seq), ctypes.byref(cs), _ptr(swa_codes),
                              _ptr(swa_scale), T_swa, _ptr(swa_start), _ptr(swa_len),
                              _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(stream, scores))
    _check(name, st)


def csa2_block_pool(scores, n_valid, n_cols, n_blocks, pool, pool_len, ws=None, block=8,
                    topk=None, stream=None):
    """pool [Q, n_blocks * block] i32, pool_len [Q] i64; topk None or
    [Q, k] i32 (the Full layer's own top-k, selected inside the pool)."""
    _dtype(scores, torch.float32, "scores"); _dtype(n_valid, torch.int64, "n_valid")
    _dtype(pool, torch.int32, "pool"); _dtype(pool_len, torch.int64, "pool_len")
    _dtype(topk, torch.int32, "topk")
    Q = scores.shape[0]
    k = topk.shape[1] if topk is not None else 0
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib().csa2_block_pool(_ptr(scores), scores.shape[1], Q, _ptr(n_valid), n_cols, block,
                               n_blocks, _ptr(pool), _ptr(pool_len), k, _ptr(topk), _ptr(ws), wsb,
                               _stream(stream, scores))
    _check("csa2_block_pool", st)


def csa2_sparse_attend(q, q_seq, cache, idx, swa_codes, swa_scale, swa_start, swa_len, out,
                       lse=None, ws=None, stream=None):
    """q [Q, 64, 512] bf16, idx [Q, k] i32 (or None with k = 0),
    swa_codes [B, T_swa, 512] u8, swa_scale [B, T_swa] f32, swa_start [Q] i64,
    swa_len [Q] i32, out [Q, 64, 512] f32, lse [Q, 64] f32 or None."""
    _dtype(q, torch.bfloat16, "q"); _dtype(q_seq, torch.int32, "q_seq")
    _dtype(idx, torch.int32, "idx"); _dtype(swa_codes, torch.uint8, "swa_codes")
    _dtype(swa_scale, torch.float32, "swa_scale"); _dtype(swa_start, torch.int64, "swa_start")
    _dtype(swa_len, torch.int32, "swa_len"); _dtype(out, torch.float32, "out")
    _dtype(lse, torch.float32, "lse")
    Q = q.shape[0]
    k = idx.shape[1] if idx is not None else 0
    T_swa = swa_codes.shape[1] if swa_codes is not None else 0
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    cs = cache.c_struct()
    st = lib().csa2_sparse_attend(_ptr(q), _ptr(q_seq), Q, ctypes.byref(cs), _ptr(idx), k,
                                  _ptr(swa_codes), _ptr(swa_scale), T_swa, _ptr(swa_start),
                                  _ptr(swa_len), _ptr(out), _ptr(lse), _ptr(ws), wsb,
                                  _stream(stream, q))
    _check("csa2_sparse_attend", st)


def csa2_selftest(device="cuda"):
    """Run the device self-test; returns the list of failure counters."""
    n = lib().csa2_selftest(None, 0, None)
    counts = torch.zeros(n, dtype=torch.int32, device=device)
    st = lib().csa2_selftest(_ptr(counts), n, _stream(None, counts))
    if st != 0:
        raise RuntimeError(f"csa2_selftest launch failed ({st})")
    torch.cuda.synchronize(counts.device)
    return counts.cpu().tolist()


def workspace(op, Q, n_cols, k, device):
    """A zero-filled uint8 device tensor of the size csa2_workspace_bytes asks
    for, or None when the operation needs none."""
    n = csa2_workspace_bytes(op, Q, n_cols, k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def csa2_decode_append(h_new, z_new, swa_new, w_ik, cache, state, n_vis=None, swa_start=None,
                       swa_len=None, stream=None):
    """h_new, z_new (None iff m == 1), swa_new: [B, 512] bf16; w_ik [128, 512]
    bf16; n_vis / swa_start [B] int64 and swa_len [B] int32 outputs or None."""
    for t, n in ((h_new, "h_new"), (z_new, "z_new"), (swa_new, "swa_new"), (w_ik, "w_ik")):
        _dtype(t, torch.bfloat16, n)
    _dtype(n_vis, torch.int64, "n_vis"); _dtype(swa_start, torch.int64, "swa_start")
    _dtype(swa_len, torch.int32, "swa_len")
    cs, ss = cache.c_struct(), state.c_struct()
    st = lib().csa2_decode_append(_ptr(h_new), _ptr(z_new), _ptr(swa_new), h_new.shape[0],
                                  _ptr(w_ik), ctypes.byref(cs), ctypes.byref(ss), _ptr(n_vis),
                                  _ptr(swa_start), _ptr(swa_len), _stream(stream, h_new))
    _check("csa2_decode_append", st)


def csa2_sparse_attend_rope(q, q_seq, cache, idx, swa_codes, swa_scale, swa_start, swa_len,
                            q_pos, dims, theta, out, lse=None, ws=None, stream=None):
    """As csa2_sparse_attend, with the query's last `dims` channels turned by
    q_pos [Q] i64 (theta^(-2i/dims) per pair) before and the output's turned
    back after; out [Q, 64, 512] bf16."""
    _dtype(q, torch.bfloat16, "q"); _dtype(q_seq, torch.int32, "q_seq")
    _dtype(idx, torch.int32, "idx"); _dtype(swa_codes, torch.uint8, "swa_codes")
    _dtype(swa_scale, torch.float32, "swa_scale"); _dtype(swa_start, torch.int64, "swa_start")
    _dtype(swa_len, torch.int32, "swa_len"); _dtype(out, torch.bfloat16, "out")
    _dtype(lse, torch.float32, "lse"); _dtype(q_pos, torch.int64, "q_pos")
    Q = q.shape[0]
    k = idx.shape[1] if idx is not None else 0
    T_swa = swa_codes.shape[1] if swa_codes is not None else 0
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    cs = cache.c_struct()
    rp = _Rope(q_pos.data_ptr() if q_pos is not None else None, dims, theta)
    st = lib().csa2_sparse_attend_rope(_ptr(q), _ptr(q_seq), Q, ctypes.byref(cs), _ptr(idx), k,
                                       _ptr(swa_codes), _ptr(swa_scale), T_swa, _ptr(swa_start),
                                       _ptr(swa_len), ctypes.byref(rp), _ptr(out), _ptr(lse),
                                       _ptr(ws), wsb, _stream(stream, q))
    _check("csa2_sparse_attend_rope", st)
