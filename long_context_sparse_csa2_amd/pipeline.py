"""One decode (or prefill) step of the CSA2 global branch, composed from the
C-ABI calls: the layer schedule of a workload run layer by layer.

Report digest "DeepSeek-V4.1-Flash", section 2.3.1: a Full layer produces
main KV and indexer K and runs the indexer; a Reindex layer rescores the
shared keys with its own indexer query and picks its own top-k; a Reuse
layer attends with the latest top-k indices and runs no indexer.  Section
2.3.2: in the decoder the first Full layer also builds the 2048 x 8 block
pool that the Reindex layers search.  Layers run one after another (layer
l + 1's queries would depend on layer l's output in the model).

A prefill step starts each chunk of queries by compressing the chunk's own
raw tokens into its entries (steps a1-a3; query i is entry i and sees
entries 0..i), so the compressor is timed with the rest of the step.

A long encoder prefill (the commentary, section 4 item 4: the encoder's
indexer stays quadratic, outside the hierarchy) runs its queries in chunks
of `q_chunk`: per chunk, every layer scores the chunk's queries against
their causally visible entries, selects and attends, so the score buffer is
q_chunk x N instead of N x N.  Each query's result does not depend on the
chunk it runs in.

Buffers are allocated once with torch; `run()` only enqueues kernels.
"""

from collections import namedtuple

import torch

from . import (Cache, CSA2_OP_ATTEND, CSA2_OP_POOL, CSA2_OP_POOL_ATTEND, CSA2_OP_SELECT_ATTEND,
               CSA2_OP_TOPK, csa2_block_pool, csa2_compress_quant, csa2_index_score,
               csa2_index_score_levels, csa2_select_attend, csa2_select_topk, csa2_sparse_attend,
               workspace)
from .synth import Workload

# one C-ABI call of a step: its name, layer, thunk and query rows [i0, i1)
Op = namedtuple("Op", "name layer fn rows")
# the calls that end a layer (its attention)
ATTEND_OPS = ("sparse_attend", "select_attend_full", "select_attend_pool")


def build_cache(wl: Workload, device, seq_chunk=1):
    """Draw each sequence's raw latents on the device and compress them into a
    fresh cache (steps a1-a3), a few sequences at a time to bound memory."""
    cache = Cache(wl.B, wl.N, device)
    w_ik = wl.w_ik(device)
    for b0 in range(0, wl.B, seq_chunk):
        b1 = min(wl.B, b0 + seq_chunk)
        h, z = wl.latents(device, b0, b1)
        sub = cache.view(b0, b1)
        csa2_compress_quant(h, z, wl.m, w_ik, sub)
        del h, z
    return cache, w_ik


class Step:
    """All layers of one step of a workload over a built cache."""

    def __init__(self, wl: Workload, device, cache=None, fp4q=False, fused=None):
        """fp4q=True scores with the MXFP4 indexer query
        (csa2_index_score_fp4q) instead of the bf16 one.  fused=True runs
        each selection together with its attention (csa2_select_attend),
        the Full layer's scan also writing the selection's lowest maxima
        levels (csa2_index_score_levels); the default does so for decode
        batches (fewer than 256 queries) and uses the separate calls for
        prefill chunks."""
        self.wl = wl
        self.device = device
        self.fp4q = fp4q
        if cache is None:
            cache, w_ik = build_cache(wl, device)
        else:
            w_ik = wl.w_ik(device)
        self.cache = cache
        self.w_ik = w_ik
        # a prefill keeps its raw latents: each chunk compresses its own tokens
        self.h = self.z = None
        if wl.prefill:
            assert wl.B == 1, "a prefill workload is one sequence"
            self.h, self.z = wl.latents(device)
        g = wl.query_geometry()
        self.q_seq = g["q_seq"].to(device)
        self.n_vis = g["n_vis"].to(device)
        self.swa_start = g["swa_start"].to(device)
        self.swa_len = g["swa_len"].to(device)
        Q, N, k = wl.Q, wl.N, wl.k
        qc = wl.q_chunk if (wl.prefill and 0 < wl.q_chunk < Q) else Q
        self.chunks = [(i0, min(Q, i0 + qc)) for i0 in range(0, Q, qc)]
        # the pool and its Reindex layers use whole-step arrays (one pool row
        # per query), so a hierarchical workload runs as one chunk
        assert not (wl.hierarchical and len(self.chunks) > 1), \
            "a hierarchical workload cannot run in query chunks"
        self.fused = (qc < 256) if fused is None else bool(fused)
        assert not (self.fused and qc >= 256), "the fused selection + attention takes < 256 queries"
        self.layers = [wl.layer_inputs(li, device) for li in range(len(wl.layers))]
        self.scores = torch.empty(qc, N, dtype=torch.float32, device=device)
        self.idx = torch.empty(qc, k, dtype=torch.int32, device=device)
        self.ws_topk = workspace(CSA2_OP_TOPK, qc, N, k, device)
        self.ws_attend = workspace(CSA2_OP_ATTEND, qc, 0, k, device)
        # per-layer inputs and outputs: every query's, or (reuse_chunk_inputs)
        # one chunk's worth that each chunk reuses
        self.reuse = wl.reuse_chunk_inputs and len(self.chunks) > 1
        R = wl.input_rows if self.reuse else Q
        self.out = [torch.empty(R, 64, 512, dtype=torch.float32, device=device) for _ in wl.layers]
        self.lse = [torch.empty(R, 64, dtype=torch.float32, device=device) for _ in wl.layers]
        self.out_kept = self.lse_kept = None
        self.idx_per_layer = [None] * len(wl.layers)
        self.scores_per_layer = [None] * len(wl.layers)
        if wl.hierarchical:
            P = wl.n_blocks * wl.block
            self.P = P
            self.pool = torch.empty(Q, P, dtype=torch.int32, device=device)
            self.pool_len = torch.empty(Q, dtype=torch.int64, device=device)
            self.ws_pool = workspace(CSA2_OP_POOL, Q, N, wl.n_blocks, device)
            self.pool_scores = torch.empty(Q, P, dtype=torch.float32, device=device)
            self.ws_topk_pool = workspace(CSA2_OP_TOPK, Q, P, k, device)
            self.idx_r = [torch.empty(Q, k, dtype=torch.int32, device=device) for _ in wl.layers]
        if self.fused:
            self.ws_sa_full = workspace(CSA2_OP_POOL_ATTEND if wl.hierarchical else CSA2_OP_SELECT_ATTEND,
                                        qc, N, k, device)
            if wl.hierarchical:
                self.ws_sa_pool = workspace(CSA2_OP_SELECT_ATTEND, Q, self.P, k, device)

    def ops(self):
        """The step as an ordered list of Op(name, layer, thunk, rows); each
        thunk enqueues one C-ABI call on the current stream.  A chunked
        prefill runs all layers for one chunk of queries before the next."""
        wl = self.wl
        out = []
        for (i0, i1) in self.chunks:
            n = i1 - i0
            rows = slice(i0, i1)
            loc = slice(0, n) if self.reuse else rows     # rows of the inputs and outputs
            # columns the chunk can see: causal prefill query i sees i + 1 entries
            n_cols = i1 if wl.prefill else wl.N
            q_seq, n_vis = self.q_seq[rows], self.n_vis[rows]
            swa_start, swa_len = self.swa_start[rows], self.swa_len[rows]
            scores, idx_full = self.scores[:n], self.idx[:n]
            idx = idx_full
            if wl.prefill:
                m = wl.m
                out.append(Op("compress", -1, lambda i0=i0, i1=i1: csa2_compress_quant(
                    self.h[:, i0 * m:i1 * m], None if self.z is None else self.z[:, i0 * m:i1 * m],
                    m, self.w_ik, self.cache, e0=i0), (i0, i1)))
            for li, mode in enumerate(wl.layers):
                L = {key: v[loc] if key in ("q_idx", "w", "q_attn") else v
                     for key, v in self.layers[li].items()}
                if mode == "full":
                    idx = idx_full
                    if self.fused:
                        # the scan also lays down the selection's lowest maxima
                        # levels; then the pool (hierarchical) or the top-k, and
                        # the attention, in one call
                        nb = wl.n_blocks if wl.hierarchical else 0
                        out.append(Op("index_score_full", li, lambda L=L, q_seq=q_seq, n_vis=n_vis,
                                      n_cols=n_cols, scores=scores, nb=nb: csa2_index_score_levels(
                            L["q_idx"], L["w"], q_seq, n_vis, n_cols, self.cache, scores,
                            self.ws_sa_full, n_blocks=nb, fp4q=self.fp4q), (i0, i1)))
                        out.append(Op("select_attend_full", li, lambda L=L, li=li, q_seq=q_seq,
                                      n_vis=n_vis, n_cols=n_cols, scores=scores, idx=idx_full,
                                      swa_start=swa_start, swa_len=swa_len, rows=loc, nb=nb:
                                      csa2_select_attend(
                            scores, n_vis, None, n_cols, wl.k, idx, L["q_attn"], q_seq, self.cache,
                            L["swa_codes"], L["swa_scale"], swa_start, swa_len,
                            self.out[li][rows], self.lse[li][rows], self.ws_sa_full, n_blocks=nb,
                            pool=self.pool if nb else None, pool_len=self.pool_len if nb else None,
                            levels=True), (i0, i1)))
                        continue
                    # (a prefill chunk's scan is bound by its MFMA and conversion
                    # work, and the maxima epilogue costs it about what the
                    # separate maxima pass does: the plain scan here)
                    out.append(Op("index_score_full", li, lambda L=L, q_seq=q_seq, n_vis=n_vis,
                                  n_cols=n_cols, scores=scores: csa2_index_score(
                        L["q_idx"], L["w"], q_seq, n_vis, None, n_cols, self.cache, scores,
                        fp4q=self.fp4q), (i0, i1)))
                    if wl.hierarchical:
                        # the pool and the layer's own top-k in one selection pass
                        out.append(Op("block_pool_topk", li, lambda: csa2_block_pool(
                            self.scores, self.n_vis, wl.N, wl.n_blocks, self.pool, self.pool_len,
                            self.ws_pool, block=wl.block, topk=self.idx), (i0, i1)))
                    else:
                        out.append(Op("select_topk_full", li, lambda n_vis=n_vis, n_cols=n_cols,
                                      scores=scores, idx=idx_full: csa2_select_topk(
                            scores, n_vis, None, n_cols, wl.k, idx, self.ws_topk), (i0, i1)))
                elif mode == "reindex":
                    idx = self.idx_r[li]
                    out.append(Op("index_score_pool", li, lambda L=L: csa2_index_score(
                        L["q_idx"], L["w"], self.q_seq, self.pool_len, self.pool, self.P,
                        self.cache, self.pool_scores, fp4q=self.fp4q), (i0, i1)))
                    if self.fused:
                        out.append(Op("select_attend_pool", li, lambda L=L, li=li, idx=idx:
                                      csa2_select_attend(
                            self.pool_scores, self.pool_len, self.pool, self.P, wl.k, idx,
                            L["q_attn"], self.q_seq, self.cache, L["swa_codes"], L["swa_scale"],
                            self.swa_start, self.swa_len, self.out[li], self.lse[li],
                            self.ws_sa_pool), (i0, i1)))
                        continue
                    out.append(Op("select_topk_pool", li, lambda idx=idx: csa2_select_topk(
                        self.pool_scores, self.pool_len, self.pool, self.P, wl.k, idx,
                        self.ws_topk_pool), (i0, i1)))
                out.append(Op("sparse_attend", li, lambda L=L, li=li, idx=idx, q_seq=q_seq,
                              swa_start=swa_start, swa_len=swa_len, rows=loc: csa2_sparse_attend(
                    L["q_attn"], q_seq, self.cache, idx, L["swa_codes"], L["swa_scale"],
                    swa_start, swa_len, self.out[li][rows], self.lse[li][rows], self.ws_attend),
                    (i0, i1)))
        return out

    def run(self, keep=False, events=None, keep_rows=None):
        """Enqueue every layer of the step.  keep=True also keeps each
        layer's indices and scores (for checking): of every query, or with
        keep_rows (ascending query ids) of those queries only, row j of the
        kept arrays then being query keep_rows[j].  `events`, a dict, gets
        (start, end) torch.cuda.Event pairs recorded around each call on the
        current stream, keyed by call name."""
        wl = self.wl
        Q = wl.Q
        kept = torch.arange(Q) if keep_rows is None else torch.as_tensor(keep_rows, dtype=torch.int64)
        nk = len(kept)
        for op in self.ops():
            name, li, (i0, i1) = op.name, op.layer, op.rows
            if events is None:
                op.fn()
            else:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                op.fn()
                e1.record()
                events.setdefault(name, []).append((e0, e1))
            if keep and name in ATTEND_OPS:
                mode = wl.layers[li]
                src_idx = self.idx_r[li] if mode == "reindex" else self.idx
                sel = ((kept >= i0) & (kept < i1)).nonzero().flatten()   # kept rows in this chunk
                dst = sel.to(self.device)
                src_rows = (kept[sel] - i0).to(self.device)
                if self.idx_per_layer[li] is None:
                    self.idx_per_layer[li] = torch.empty(nk, wl.k, dtype=torch.int32,
                                                         device=self.device)
                self.idx_per_layer[li][dst] = src_idx.index_select(0, src_rows)
                if self.reuse:                  # outputs are overwritten by the next chunk
                    if self.out_kept is None:
                        self.out_kept = [torch.empty(nk, 64, 512, device=self.device) for _ in wl.layers]
                        self.lse_kept = [torch.empty(nk, 64, device=self.device) for _ in wl.layers]
                    self.out_kept[li][dst] = self.out[li].index_select(0, src_rows)
                    self.lse_kept[li][dst] = self.lse[li].index_select(0, src_rows)
                if mode in ("full", "reindex"):
                    src = self.scores if mode == "full" else self.pool_scores
                    if self.scores_per_layer[li] is None:
                        self.scores_per_layer[li] = torch.empty(nk, src.shape[1], dtype=torch.float32,
                                                                device=self.device)
                    self.scores_per_layer[li][dst] = src.index_select(0, src_rows)

    def scan_index(self):
        """Position of the (first) Full-layer scan among the step's calls."""
        return next(i for i, op in enumerate(self.ops()) if op.name == "index_score_full")

    def capture(self, split_first=True):
        """Capture the step into HIP graphs: [the calls before the first
        scan] (when there are any), [that scan] and [the rest] (split_first),
        or one graph.  Returns the list of graphs; replaying them in order is
        one step."""
        ops = self.ops()
        if split_first:
            i = self.scan_index()
            groups = ([ops[:i]] if i > 0 else []) + [ops[i:i + 1], ops[i + 1:]]
        else:
            groups = [ops]
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for grp in groups:              # one eager pass on the capture stream first
                for op in grp:
                    op.fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for grp in groups:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for op in grp:
                    op.fn()
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs
