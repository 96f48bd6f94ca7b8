"""The five workloads at their full sizes, in the launch configuration
bench.py times, checked against the fp64 oracle stage by stage (each oracle
stage takes the GPU's previous-stage result as input).  Every score, every
selection and every attention output is compared; only the compression of
the decode caches (built before the step, not timed) is checked on a seeded
sample of entries.

c0  N = 2048, batch 1.
c1  batch 32 x N = 65,536.
c2  batch 4 x N = 2^20, Full + pool + 4 Reindex: all 2^20 fp64 scores of
    every query, the Full top-512 and the 2048-block pool against the fp64
    ranking (near-ties only may swap), every Reindex score and selection.
c3  prefill, 8192 raw -> 4096 entries (m = 2), 4096 causal queries: every
    score and every top-k; attention on a sample of queries.
c4  batch 8 x 2^19 entries from 2^20 raw (m = 2), Full + 5 Reuse: all fp64
    scores, the Full top-512 against the fp64 ranking, every attention
    output.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_csa2_amd import synth
from long_context_sparse_csa2_amd.pipeline import Step
from oracle import csa2_ref as R
from tests import checks

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check_compression_sample(wl, cache, w_ik, n_sample, seed):
    """Regenerate each sampled sequence's raw latents (same device and seed)
    and compare sampled entries of a1-a3 with the oracle."""
    rng = np.random.default_rng(seed)
    w64 = checks.bf16_to_f64(w_ik)
    for b in sorted(set(rng.integers(0, wl.B, 2).tolist()) | {wl.B - 1}):
        h, z = wl.latents(DEV, b, b + 1)
        ent = np.sort(rng.choice(wl.N, min(n_sample, wl.N), replace=False))
        ent[-1] = wl.N - 1
        rows = (ent[:, None] * wl.m + np.arange(wl.m)[None, :]).reshape(-1)
        rows_t = torch.from_numpy(rows).to(DEV)
        h64 = checks.bf16_to_f64(h[0].index_select(0, rows_t))
        z64 = checks.bf16_to_f64(z[0].index_select(0, rows_t)) if z is not None else None
        del h, z
        x = R.compress(h64, z64, wl.m)
        hmax = np.abs(h64).reshape(-1, wl.m, 512).max(1)
        e_t = torch.from_numpy(ent).to(DEV)
        kv_c = checks.host(cache.kv_codes[b].index_select(0, e_t))
        kv_s = checks.host(cache.kv_scales[b].index_select(0, e_t))
        checks.check_main_kv(x, wl.m, kv_c, kv_s, hmax)
        checks.check_indexer_k(kv_c, kv_s, w64, checks.host(cache.ik_codes[b].index_select(0, e_t)),
                               checks.host(cache.ik_scales[b].index_select(0, e_t)))


def _run(name):
    wl = synth.WORKLOADS[name]
    step = Step(wl, DEV)
    step.run(keep=True)
    torch.cuda.synchronize()
    return wl, step


def test_c1_batched_full_decode():
    wl, step = _run("c1")
    _check_compression_sample(wl, step.cache, wl.w_ik(DEV), 512, seed=1)
    checks.check_step(step)


def test_c2_hierarchical_1m_decode():
    wl, step = _run("c2")
    _check_compression_sample(wl, step.cache, wl.w_ik(DEV), 512, seed=2)
    checks.check_step(step)
    # the Full layer's own top-512 lies inside its pool (report section 2.3.2)
    pool = checks.host(step.pool)
    full_idx = checks.host(step.idx_per_layer[0])
    for q in range(wl.Q):
        assert set(full_idx[q].tolist()) <= set(pool[q].tolist())
        assert int(checks.host(step.pool_len[q])) == 16384


def test_c3_prefill_m2():
    wl, step = _run("c3")
    _check_compression_sample(wl, step.cache, wl.w_ik(DEV), 4096, seed=3)
    L = step.layers[0]
    q64 = checks.bf16_to_f64(L["q_idx"])
    w64 = checks.host(L["w"]).astype(np.float64)
    khat = R.dequant_mxfp4(checks.host(step.cache.ik_codes[0]), checks.host(step.cache.ik_scales[0]))
    s_gpu = checks.host(step.scores_per_layer[0])
    idx = checks.host(step.idx_per_layer[0])
    for q0 in range(0, wl.Q, 256):
        dots = np.einsum("ec,qhc->qeh", khat, q64[q0:q0 + 256])
        ref = np.einsum("qeh,qh->qe", np.maximum(dots, 0), w64[q0:q0 + 256])
        for i in range(ref.shape[0]):
            q = q0 + i
            nv = q + 1
            checks.check_scores(s_gpu[q, :nv], ref[i, :nv])
            checks.check_topk_exact(idx[q], s_gpu[q, :nv], wl.k)
            checks.check_topk_tolerance(idx[q], ref[i, :nv], wl.k)
    sample = sorted({0, 1, 2, 63, 64, 511, 512, 513, wl.Q - 1} | set(np.random.default_rng(3).integers(0, wl.Q, 24).tolist()))
    checks.check_step(step, q_sample=sample)


def test_c4_reuse_decode_m2():
    wl, step = _run("c4")
    _check_compression_sample(wl, step.cache, wl.w_ik(DEV), 512, seed=4)
    checks.check_step(step)
    # Reuse layers attend over the Full layer's indices
    for li in range(1, len(wl.layers)):
        assert torch.equal(step.idx_per_layer[li], step.idx_per_layer[0])
