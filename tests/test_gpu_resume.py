"""Checkpoint and resume: the 356 B/entry cache (commentary, section 2) and
the per-sequence decode state (V4 page, Fig. 6: SWA rows and the
uncompressed tail) are the layer's whole state, so copying them to the host
and back reproduces the next step bit for bit."""
import math

import pytest
import torch

import long_context_sparse_csa2_amd as C
from long_context_sparse_csa2_amd import synth
from long_context_sparse_csa2_amd.pipeline import Step

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _outputs(step):
    wl = step.wl
    step.run(keep=True)
    torch.cuda.synchronize()
    o = {f"out{li}": step.out[li].clone() for li in range(len(wl.layers))}
    o.update({f"lse{li}": step.lse[li].clone() for li in range(len(wl.layers))})
    o.update({f"idx{li}": step.idx_per_layer[li].clone() for li in range(len(wl.layers))})
    o.update({f"scores{li}": step.scores_per_layer[li].clone()
              for li in range(len(wl.layers)) if step.scores_per_layer[li] is not None})
    if wl.hierarchical:
        o["pool"], o["pool_len"] = step.pool.clone(), step.pool_len.clone()
    return o


def test_cache_round_trip_through_host_gives_the_same_step():
    """A hierarchical decode step (Full + pool + 2 Reindex) before and after
    the cache went to the host and came back into memory overwritten with
    other bytes in between."""
    wl = synth.scaled(synth.WORKLOADS["c2"], B=2, T=60000, layers=["full", "reindex", "reindex"])
    step = Step(wl, DEV)
    a = _outputs(step)
    saved = {k: v.cpu() for k, v in step.cache.arrays().items()}
    for v in step.cache.arrays().values():
        v.fill_(0xAB)
    for k, v in step.cache.arrays().items():
        v.copy_(saved[k].to(DEV))
    b = _outputs(step)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_decode_state_resume():
    """m = 2, W = 16: 41 tokens appended, then the cache and the state block
    saved to the host; 9 more tokens and a decode query (scores, top-8,
    attention over the selection and the SWA ring) run on the live buffers
    and again on fresh buffers restored from the saved bytes: identical."""
    B, m, W, cap = 2, 2, 16, 40
    g = torch.Generator().manual_seed(11)
    h = (torch.randn(B, 50, 512, generator=g)).to(torch.bfloat16).to(DEV)
    z = (torch.randn(B, 50, 512, generator=g) * 2).to(torch.bfloat16).to(DEV)
    sw = (torch.randn(B, 50, 512, generator=g)).to(torch.bfloat16).to(DEV)
    w_ik = (torch.randn(128, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16).to(DEV)
    qi = torch.randn(B, 32, 128, generator=g).to(torch.bfloat16).to(DEV)
    wq = torch.rand(B, 32, generator=g).to(DEV)
    qa = (torch.randn(B, 64, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16).to(DEV)
    q_seq = torch.arange(B, dtype=torch.int32, device=DEV)

    def fresh():
        cache, st = C.Cache(B, cap, DEV), C.State(B, m, W, DEV)
        for v in cache.arrays().values():
            v.fill_(0)
        return cache, st

    def append(cache, st, t0, t1):
        n_vis = torch.zeros(B, dtype=torch.int64, device=DEV)
        s0 = torch.zeros(B, dtype=torch.int64, device=DEV)
        sl = torch.zeros(B, dtype=torch.int32, device=DEV)
        for t in range(t0, t1):
            C.csa2_decode_append(h[:, t].contiguous(), z[:, t].contiguous(), sw[:, t].contiguous(),
                                 w_ik, cache, st, n_vis, s0, sl)
        return n_vis, s0, sl

    def query(cache, st, n_vis, s0, sl):
        scores = torch.empty(B, cap, device=DEV)
        C.csa2_index_score(qi, wq, q_seq, n_vis, None, cap, cache, scores)
        idx = torch.empty(B, 8, dtype=torch.int32, device=DEV)
        C.csa2_select_topk(scores, n_vis, None, cap, 8, idx, C.workspace(C.CSA2_OP_TOPK, B, cap, 8, DEV))
        out = torch.empty(B, 64, 512, device=DEV)
        lse = torch.empty(B, 64, device=DEV)
        C.csa2_sparse_attend(qa, q_seq, cache, idx, st.swa_codes, st.swa_scale, s0, sl, out, lse,
                             C.workspace(C.CSA2_OP_ATTEND, B, 0, 8, DEV))
        torch.cuda.synchronize()
        return [n_vis, s0, sl, scores.nan_to_num(0.0) * (torch.arange(cap, device=DEV) < n_vis[:, None]),
                idx, out, lse]

    cache, st = fresh()
    append(cache, st, 0, 41)
    torch.cuda.synchronize()
    saved_c = {k: v.cpu() for k, v in cache.arrays().items()}
    state_names = ("tail_h", "tail_z", "n_tok", "swa_codes", "swa_scale")
    saved_s = {k: getattr(st, k).cpu() for k in state_names}
    live = query(cache, st, *append(cache, st, 41, 50))
    cache2, st2 = fresh()
    for k, v in cache2.arrays().items():
        v.copy_(saved_c[k].to(DEV))
    for k in state_names:
        getattr(st2, k).copy_(saved_s[k].to(DEV))
    resumed = query(cache2, st2, *append(cache2, st2, 41, 50))
    for a, b in zip(live, resumed):
        assert torch.equal(a, b)
