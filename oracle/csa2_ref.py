"""fp64 reference for every step of the CSA2 global branch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

One function per step, each a direct transcription of the definition, in
float64, with numpy primitives (matmul, lexsort) as the only library help.
Nothing is blocked, fused or reordered.  Where the pages leave a detail open
the reading taken is stated in the function's docstring.

Cache layout (one KV-producing layer, per entry, structure of arrays):
  kv_codes  [.., 256] u8   E2M1 main-KV codes, channel 2c in the low nibble
  kv_scales [.., 32]  u8   E4M3FN scale of channels 16g .. 16g+15
  ik_codes  [.., 64]  u8   E2M1 indexer-K codes, dim 2c in the low nibble
  ik_scales [.., 4]   u8   E8M0 scale of dims 32g .. 32g+31
which is 256 + 32 + 64 + 4 = 356 bytes per entry (mer.dev commentary,
section 2: 288 B main KV + 68 B indexer K).
"""

import numpy as np

from . import formats as F

D_LATENT = 512          # main-KV latent width (commentary, section 1 setup)
KV_GROUP = 16           # channels per E4M3 scale (report, section 2.4.4)
D_INDEX = 128           # indexer head dim (commentary, section 1 setup)
MX_GROUP = 32           # elements per E8M0 scale (OCP MXFP4)
H_INDEX = 32            # indexer heads
H_ATTN = 64             # attention query heads


# ------------------------------------------------------------ a1 compressor
def compress(h, z, m):
    """Non-overlapping m-to-1 softmax-weighted pooling.

    The report (section 2.3) says CSA2 drops the overlap between the source
    entries of adjacent compressed entries and drops the absolute position
    embedding; the commentary (section 4.1) fills the pooling in as a softmax
    weighting following DSA/V4.  Reading: per channel c, entry j is
        x[j, c] = sum_t softmax_t(z[jm+t, c]) * h[jm+t, c],  t = 0..m-1,
    with the compression logits z of the same shape as the latents h
    (Eq. 1 of the report gives C and Z the same shape).  For m = 1 the
    softmax of a single logit is 1, so x = h.
    """
    h = np.asarray(h, dtype=np.float64)
    T, C = h.shape
    assert T % m == 0
    if m == 1:
        return h.copy()
    z = np.asarray(z, dtype=np.float64)
    hh = h.reshape(T // m, m, C)
    zz = z.reshape(T // m, m, C)
    e = np.exp(zz - zz.max(axis=1, keepdims=True))
    return (e * hh).sum(axis=1) / e.sum(axis=1)


# ------------------------------------------------------ a2 main-KV FP4 quant
def quant_main_kv(x):
    """E2M1 elements with one E4M3FN scale per 16 channels, no global scale
    (report section 2.4.4, following NVFP4 minus its second-level scale; the
    commentary's formula for a 16-channel group was lost in extraction).
    Reading: s = RNE_E4M3FN(max|x_g| / 6) with saturation; if s == 0 every
    code is +0, else code = RNE_E2M1(x / s) saturating at +-6.
    Returns (codes [n, 256] u8, scales [n, 32] u8)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    g = x.reshape(n, D_LATENT // KV_GROUP, KV_GROUP)
    amax = np.abs(g).max(axis=2)
    sc = F.e4m3fn_encode(amax / 6.0)
    s = F.e4m3fn_value(sc)[:, :, None]
    safe = np.where(s > 0, s, 1.0)
    codes = np.where(s > 0, F.e2m1_encode(g / safe), 0).astype(np.uint8)
    return F.pack_nibbles(codes.reshape(n, D_LATENT)), sc.astype(np.uint8)


def dequant_main_kv(codes, scales):
    """[.., 256] codes + [.., 32] E4M3FN scales -> fp64 [.., 512]."""
    v = F.e2m1_value(F.unpack_nibbles(codes))
    s = F.e4m3fn_value(scales)
    shp = v.shape[:-1]
    return (v.reshape(shp + (D_LATENT // KV_GROUP, KV_GROUP)) * s[..., None]).reshape(shp + (D_LATENT,))


# ------------------------------------------- a3 indexer-K projection + MXFP4
def project_indexer_k(xhat, w_ik):
    """Indexer K is a linear projection of the stored main-KV entry (report
    section 2.3: 'obtains indexer K by projecting main KV entries').  Reading:
    the projection reads the dequantised FP4 main KV, the value the cache
    holds.  w_ik is [128, 512] (output dim x input channel), so
    k[j, d] = sum_c w_ik[d, c] * xhat[j, c]."""
    return np.asarray(xhat, dtype=np.float64) @ np.asarray(w_ik, dtype=np.float64).T


def quant_mxfp4(k):
    """OCP MXFP4: per block of 32, X = 2^(floor(log2 max|k|) - 2) stored as
    E8M0 (exponent clamped to [-127, 127]); elements RNE_E2M1(k / X)
    saturating at +-6.  An all-zero block stores scale byte 0 and codes +0.
    Returns (codes [n, 64] u8, scales [n, 4] u8)."""
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    g = k.reshape(n, D_INDEX // MX_GROUP, MX_GROUP)
    amax = np.abs(g).max(axis=2)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex, f in [0.5, 1)
    E = np.clip(ex - 1 - 2, -127, 127)     # floor(log2 amax) - emax(E2M1)
    E = np.where(amax > 0, E, -127)
    X = np.exp2(E.astype(np.float64))[:, :, None]
    codes = np.where(amax[:, :, None] > 0, F.e2m1_encode(g / X), 0).astype(np.uint8)
    return F.pack_nibbles(codes.reshape(n, D_INDEX)), (E + 127).astype(np.uint8)


def dequant_mxfp4(codes, scales):
    """[.., 64] codes + [.., 4] E8M0 scales -> fp64 [.., 128]."""
    v = F.e2m1_value(F.unpack_nibbles(codes))
    s = F.e8m0_value(scales)
    shp = v.shape[:-1]
    return (v.reshape(shp + (D_INDEX // MX_GROUP, MX_GROUP)) * s[..., None]).reshape(shp + (D_INDEX,))


def build_entries(h, z, m, w_ik):
    """Steps a1-a3 for one sequence: raw latents [T, 512] (+ logits) -> the
    four cache arrays of T/m entries, plus the fp64 values the quantisers saw
    (pooled x and projected k), which the tests use to measure margins."""
    x = compress(h, z, m)
    kv_c, kv_s = quant_main_kv(x)
    xhat = dequant_main_kv(kv_c, kv_s)
    k = project_indexer_k(xhat, w_ik)
    ik_c, ik_s = quant_mxfp4(k)
    return dict(kv_codes=kv_c, kv_scales=kv_s, ik_codes=ik_c, ik_scales=ik_s, x=x, k=k)


# ------------------------------------------------------------ a4 index score
def index_scores(q_idx, w, khat):
    """Lightning-indexer score of one query against entries:
        s_j = sum_h w_h * max(0, q_h . k_j)
    over 32 heads of dim 128 (commentary section 4.1 fills in this
    ReLU-weighted multi-head form following DSA/V4; no extra scale factor).
    q_idx [32, 128], w [32], khat [n, 128] -> fp64 [n]."""
    q = np.asarray(q_idx, dtype=np.float64)
    dots = np.asarray(khat, dtype=np.float64) @ q.T          # [n, 32]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# ------------------------------------------------- f1 MXFP4 indexer query
def quant_indexer_q(q_idx):
    """MXFP4 form of the indexer query.  The report (section 2.4.4) says V4
    already trains the indexer queries and keys for OCP MXFP4 so that the
    index product runs as an FP4 matrix multiply; the commentary (section 5)
    repeats it.  Reading: the rule of quant_mxfp4 (the OCP MX rule used for
    the indexer K), applied per head to each 32-dim block of the bf16 query
    as given.  [.., 32, 128] -> (codes [.., 32, 64] u8, scales [.., 32, 4] u8)."""
    q = np.asarray(q_idx, dtype=np.float64)
    c, s = quant_mxfp4(q.reshape(-1, D_INDEX))
    return c.reshape(q.shape[:-1] + (D_INDEX // 2,)), s.reshape(q.shape[:-1] + (D_INDEX // MX_GROUP,))


def index_scores_fp4q(q_idx, w, khat):
    """Step a4 with the MXFP4 query: index_scores of the dequantised
    quant_indexer_q(q_idx) against the dequantised indexer K.
    q_idx [32, 128], w [32], khat [n, 128] -> fp64 [n]."""
    c, s = quant_indexer_q(q_idx)
    return index_scores(dequant_mxfp4(c, s), w, khat)


# ---------------------------------------------------------------- a5 top-k
def topk(scores, k, ids=None):
    """The min(k, n) candidates with the largest score; ties broken towards
    the lower entry id.  Returns the selected ids, ascending (the result is
    a set)."""
    s = np.asarray(scores, dtype=np.float64)
    ids = np.arange(s.size, dtype=np.int64) if ids is None else np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -s))
    return np.sort(ids[order[:min(k, s.size)]])


def kth_score(scores, k):
    """Score of the k-th best candidate (the last one selected)."""
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    return s[min(k, s.size) - 1]


# ------------------------------------------------------------ a6 block pool
def block_pool(scores, block=8, n_blocks=2048):
    """Hierarchical Sparse Indexer candidate pool (report section 2.3.2 and
    Fig. 5; commentary section 4.3): each aligned block of `block` positions
    gets the maximum score among its visible positions, the blocks are ranked
    by (max desc, block id asc), the first min(n_blocks, #blocks) are kept,
    and the pool is the visible positions they cover, ascending.  `scores`
    holds the n_vis visible entries; a partial last block uses its visible
    members only."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    nb = (n + block - 1) // block
    pad = np.full(nb * block, -np.inf)
    pad[:n] = s
    bmax = pad.reshape(nb, block).max(axis=1)
    order = np.lexsort((np.arange(nb), -bmax))
    keep = np.sort(order[:min(n_blocks, nb)])
    pos = (keep[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < n]


def block_max(scores, block=8):
    s = np.asarray(scores, dtype=np.float64)
    nb = (s.size + block - 1) // block
    pad = np.full(nb * block, -np.inf)
    pad[:s.size] = s
    return pad.reshape(nb, block).max(axis=1)


# ------------------------------------------------------- a8/a9 attention
def decode_swa(codes, scale):
    """FP8 SWA rows: E4M3FN codes [r, 512] times a per-row fp32 scale."""
    return F.e4m3fn_value(codes) * np.asarray(scale, dtype=np.float64).reshape(-1, 1)


def attend(q, rows):
    """Attention of 64 heads over gathered latent rows used as both key and
    value (MLA-style shared latent; report section 2.3, commentary 4.1):
        l_hj = q_h . v_j,  p_h = softmax_j(l_h),  o_h = sum_j p_hj v_j,
        lse_h = log sum_j exp(l_hj).
    The 1/sqrt(512) softmax scale is already folded into q (the workload
    draws q as N(0,1)/sqrt(512)); no sink, no further scale.
    q [64, 512], rows [r, 512] -> (o [64, 512], lse [64])."""
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(rows, dtype=np.float64)
    l = q @ v.T
    mx = l.max(axis=1, keepdims=True)
    p = np.exp(l - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p @ v) / den, (mx + np.log(den)).reshape(-1)


def gather_rows(kv_codes, kv_scales, idx, swa_codes=None, swa_scale=None):
    """Step a8: the dequantised main-KV rows of the selected entries
    (idx == -1 skipped) followed by the decoded SWA rows."""
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    rows = [dequant_main_kv(kv_codes[idx], kv_scales[idx])]
    if swa_codes is not None and len(swa_codes):
        rows.append(decode_swa(swa_codes, swa_scale))
    return np.concatenate(rows, axis=0)


# ------------------------------------- f2 decode-time append and state
SWA_WINDOW = 128        # n_win: SWA rows kept per sequence (commentary section 1 setup)


def quant_swa_row(x):
    """FP8 SWA row: E4M3FN codes with one fp32 scale per row.  The V4 page
    (Fig. 6, KV cache layout) keeps the SWA entries of the most recent
    n_win tokens in each request's state block; the pages name the format
    only as FP8.  Reading: the row scale sigma = max|x| / 448 is stored as
    an fp32 number (the exact quotient rounded to nearest, ties to even),
    and each code is RNE_E4M3FN(x / sigma) of the exact quotient by that
    stored scale, saturating at 448, so that sigma * e best approximates x;
    an all-zero row stores sigma = 0 and +0 codes.  Evaluated in fp64.
    x [.., 512] -> (codes [.., 512] u8, sigma [..] fp32)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    sig = np.asarray(amax / 448.0).astype(np.float32)        # the stored fp32 scale
    s64 = sig.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    codes = np.where(s64[..., None] > 0, F.e4m3fn_encode(x / safe[..., None]), 0)
    return codes.astype(np.uint8), sig


def new_state(m, W=SWA_WINDOW):
    """Per-sequence state block (V4 page, Fig. 6): the raw latents and
    compression logits of the tokens of a not yet complete group of m, the
    SWA ring of the last W tokens, and the token count."""
    return dict(m=m, W=W, n_tok=0,
                tail_h=np.zeros((max(m - 1, 1), D_LATENT)), tail_z=np.zeros((max(m - 1, 1), D_LATENT)),
                swa_codes=np.zeros((W, D_LATENT), np.uint8), swa_scale=np.zeros(W, np.float32))


def append_token(state, cache, h, z, swa_x, w_ik):
    """One decode token of one sequence.  Reading of the V4 page's Fig. 6:
    token t (= the count so far) waits in the tail until it completes its
    group of m; the m-th token's arrival compresses the group (steps a1-a3,
    build_entries) into entry t // m of `cache` (a dict of the four entry
    arrays, preallocated); every token's SWA row goes to ring slot t mod W.
    h, z [512] (z ignored for m = 1), swa_x [512]; updates both in place."""
    m, W, t = state["m"], state["W"], state["n_tok"]
    s = t % m
    if s == m - 1:
        hh = np.concatenate([state["tail_h"][:m - 1], np.asarray(h, np.float64)[None]], axis=0)
        zz = None if m == 1 else np.concatenate([state["tail_z"][:m - 1], np.asarray(z, np.float64)[None]], axis=0)
        e = build_entries(hh, zz, m, w_ik)
        for key in ("kv_codes", "kv_scales", "ik_codes", "ik_scales"):
            cache[key][t // m] = e[key][0]
    else:
        state["tail_h"][s] = h
        state["tail_z"][s] = z
    c, sg = quant_swa_row(swa_x)
    state["swa_codes"][t % W] = c
    state["swa_scale"][t % W] = sg
    state["n_tok"] = t + 1


def decode_geometry(n_tok, m, W=SWA_WINDOW):
    """What the next decode query of a sequence with n_tok tokens sees:
    entries 0 .. n_tok // m - 1 (the complete groups; entry j covers tokens
    jm .. jm + m - 1) and the SWA rows of the last min(W, n_tok) tokens,
    which start at ring slot (n_tok - len) mod W.  -> (n_vis, swa_start, swa_len)."""
    swa_len = min(W, n_tok)
    return n_tok // m, (n_tok - swa_len) % W if W else 0, swa_len


def swa_window(swa_codes, swa_scale, start, length):
    """The SWA ring rows start, start + 1, ... (mod W), oldest first."""
    W = len(swa_scale)
    idx = (start + np.arange(length)) % W if length > 0 else np.zeros(0, np.int64)
    return swa_codes[idx], swa_scale[idx]


# ------------------------------------ f4 RoPE around attention, bf16 cast
def rope_rotate(x, pos, dims, theta):
    """RoPE on the last `dims` of the 512 channels of each row.  Reading (the
    pages fix neither the channels, the pairing nor the base): the RoFormer
    rule on adjacent pairs, pair i = channels (512 - dims + 2i, 512 - dims +
    2i + 1) turned by the angle pos * theta^(-2i / dims):
        (a, b) -> (a cos - b sin, a sin + b cos).
    x [.., 512]; pos a scalar (one position for all rows) -> fp64 [.., 512]."""
    x = np.array(x, dtype=np.float64, copy=True)
    if dims == 0:
        return x
    i = np.arange(dims // 2)
    ang = float(pos) * np.asarray(theta, dtype=np.float64) ** (-2.0 * i / dims)
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., D_LATENT - dims::2].copy()
    b = x[..., D_LATENT - dims + 1::2].copy()
    x[..., D_LATENT - dims::2] = a * c - b * s
    x[..., D_LATENT - dims + 1::2] = a * s + b * c
    return x


def bf16_round(x):
    """Round to bf16 (8 significant bits), to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def attend_rope(q, rows, pos, dims, theta):
    """Fused RoPE - attention - inverse RoPE - cast, as the report (section
    3.2) names FlashMLA's kernel.  The cache holds post-RoPE latents (section
    2.4.4: quantised after RoPE), so the rows are used as stored; the query's
    RoPE channels are turned by its position first; the output, a
    probability-weighted mix of rows that carry their own rotations, has its
    RoPE channels turned back by the query's position (reading: the second
    RoPE of the fused kernel is this inverse rotation); the result is cast to
    bf16.  -> (o_bf16 [64, 512] as fp64, o before the cast, lse [64])."""
    o, lse = attend(rope_rotate(q, pos, dims, theta), rows)
    o = rope_rotate(o, -float(pos), dims, theta)
    return bf16_round(o), o, lse


# ----------------------------------------- layer schedule (accounting model)
ENCODER_GROUPS = 3          # each: 1 Full + 5 Reuse, m = 2
DECODER_GROUPS = 5          # first: 1 Full + 3 Reuse; then 4 x (1 Reindex + 3 Reuse), m = 1


def layer_schedule():
    """The 38 CSA2 layers of the 40-layer model, as the commentary (section
    2) lays them out: layers 0-1 are SWA only; the encoder has 3 groups of
    (Full + 5 Reuse) at m = 2, the decoder 5 groups of 4 layers at m = 1,
    the first (Full + 3 Reuse), the rest (Reindex + 3 Reuse).
    Returns [(layer, mode, m)]."""
    out, layer = [], 2
    for _ in range(ENCODER_GROUPS):
        out.append((layer, "full", 2)); layer += 1
        for _ in range(5):
            out.append((layer, "reuse", 2)); layer += 1
    for g in range(DECODER_GROUPS):
        out.append((layer, "full" if g == 0 else "reindex", 1)); layer += 1
        for _ in range(3):
            out.append((layer, "reuse", 1)); layer += 1
    return out


def entry_bytes():
    """Bytes per global-KV entry of one KV-producing layer."""
    main = D_LATENT // 2 + D_LATENT // KV_GROUP          # codes + E4M3 scales
    idx = D_INDEX // 2 + D_INDEX // MX_GROUP             # codes + E8M0 scales
    return main, idx, main + idx


def global_kv_bytes_per_token():
    """Sum over Full-mode layers of entry bytes / m: only Full layers keep
    a cache; Reindex and Reuse layers read the latest Full layer's."""
    _, _, e = entry_bytes()
    return sum(e / m for (_, mode, m) in layer_schedule() if mode == "full")


def indexer_macs_per_decode_token(n_tokens, pool=16384, hierarchical=True):
    """MACs spent by the indexers of one decode token with n_tokens of
    context: every Full layer scores each of its n_tokens/m visible entries,
    every Reindex layer scores the pool (or all entries without the
    hierarchy); a (query, entry) pair costs H_INDEX * D_INDEX MACs."""
    per_pair = H_INDEX * D_INDEX
    total = 0
    for (_, mode, m) in layer_schedule():
        if mode == "full":
            total += per_pair * n_tokens / m
        elif mode == "reindex":
            total += per_pair * (pool if hierarchical else n_tokens / m)
    return total
