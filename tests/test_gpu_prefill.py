"""Long encoder prefill in query chunks (the commentary, section 4 item 4:
the encoder's indexer scores every causally visible entry, so a long
prefill runs its queries in chunks).  A query's scores, selection and
attention must not depend on the chunk it runs in, and every stage is
checked against the fp64 oracle on sampled queries, at a small size and at
65,536 raw tokens (one encoder group: Full + 5 Reuse, m = 2, 4096-query
chunks), the configuration `bench.py --config p64k` times."""
import numpy as np
import pytest
import torch

from long_context_sparse_csa2_amd import synth
from long_context_sparse_csa2_amd.pipeline import Step
from oracle import csa2_ref as R
from tests import checks

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _small(q_chunk):
    # 4000 raw -> 2000 entries and queries; chunks of 512 (the last one 464)
    return synth.scaled(synth.WORKLOADS["p64k"], T=4000, q_chunk=q_chunk, layers=["full", "reuse"])


def test_chunked_equals_one_launch():
    wl = _small(512)
    step = Step(wl, DEV)
    assert len(step.chunks) == 4 and step.chunks[-1] == (1536, 2000)
    step.run(keep=True)
    one = Step(_small(0), DEV, cache=step.cache)
    assert len(one.chunks) == 1
    one.run(keep=True)
    torch.cuda.synchronize()
    s_a, s_b = checks.host(step.scores_per_layer[0]), checks.host(one.scores_per_layer[0])
    tri = np.tril(np.ones((wl.Q, wl.N), dtype=bool))                # query i sees entries 0..i
    assert np.array_equal(s_a[tri], s_b[tri])
    for li in range(len(wl.layers)):
        assert np.array_equal(checks.host(step.idx_per_layer[li]), checks.host(one.idx_per_layer[li]))
        assert np.array_equal(checks.host(step.out[li]), checks.host(one.out[li]))
        assert np.array_equal(checks.host(step.lse[li]), checks.host(one.lse[li]))


def test_chunked_prefill_against_oracle():
    wl = _small(512)
    step = Step(wl, DEV)
    step.run(keep=True)
    torch.cuda.synchronize()
    sample = [0, 1, 63, 511, 512, 513, 1023, 1535, 1536, 1999] + \
        np.random.default_rng(5).integers(0, wl.Q, 12).tolist()
    checks.check_step(step, q_sample=sorted(set(sample)))


def test_p64k_sampled_against_oracle():
    """Full size: scores of sampled queries against the oracle over all
    their visible entries, the exact top-512 of the GPU's scores, and every
    layer's attention over the GPU's selection."""
    wl = synth.WORKLOADS["p64k"]
    step = Step(wl, DEV)
    keep = sorted({0, 1, 4095, 4096, 4097, 16383, 16384, 32767} |
                  set(np.random.default_rng(6).integers(0, wl.Q, 8).tolist()))
    step.run(keep=True, keep_rows=keep)
    torch.cuda.synchronize()
    ik_c, ik_s = checks.host(step.cache.ik_codes[0]), checks.host(step.cache.ik_scales[0])
    kv_c, kv_s = checks.host(step.cache.kv_codes[0]), checks.host(step.cache.kv_scales[0])
    khat = R.dequant_mxfp4(ik_c, ik_s)
    s0, sl = checks.host(step.swa_start), checks.host(step.swa_len)
    s_gpu = checks.host(step.scores_per_layer[0])
    idx = checks.host(step.idx_per_layer[0])
    L0 = step.layers[0]
    for j, q in enumerate(keep):
        nv = q + 1
        ref = R.index_scores(checks.bf16_to_f64(L0["q_idx"][q]), checks.host(L0["w"][q]).astype(np.float64),
                             khat[:nv])
        checks.check_scores(s_gpu[j, :nv], ref)
        checks.check_topk_exact(idx[j], s_gpu[j, :nv], wl.k)
        checks.check_topk_tolerance(idx[j], ref, wl.k)
        for li in range(len(wl.layers)):
            assert np.array_equal(checks.host(step.idx_per_layer[li])[j], idx[j])   # Reuse layers
            L = step.layers[li]
            sc, ss = checks.swa_rows(checks.host(L["swa_codes"][0]), checks.host(L["swa_scale"][0]).astype(np.float64),
                                     int(s0[q]), int(sl[q]))
            rows = R.gather_rows(kv_c, kv_s, idx[j], sc, ss)
            checks.check_attention(checks.host(step.out[li][q]), checks.host(step.lse[li][q]),
                                   checks.bf16_to_f64(L["q_attn"][q]), rows)


def test_p1m_sampled_against_oracle():
    """The 1,048,576-raw-token end of the chunked prefill (2^19 queries in
    128 chunks of 4096; one chunk's queries reused by every chunk): sampled
    queries across the causal range -- scores against the oracle over all
    their visible entries (up to 2^19), the exact top-512 of the GPU's
    scores and its fp64 ranking within the tie bar, and every layer's
    attention over the GPU's selection."""
    wl = synth.WORKLOADS["p1m"]
    step = Step(wl, DEV)
    assert step.reuse and len(step.chunks) == 128
    keep = sorted({0, 511, 4095, 4096, 262143, 262144, wl.Q - 1} |
                  set(np.random.default_rng(7).integers(0, wl.Q, 4).tolist()))
    print(f"[p1m] step with {len(step.chunks)} chunks, checking queries {keep}", flush=True)
    step.run(keep=True, keep_rows=keep)
    torch.cuda.synchronize()
    ik_c, ik_s = checks.host(step.cache.ik_codes[0]), checks.host(step.cache.ik_scales[0])
    kv_c, kv_s = checks.host(step.cache.kv_codes[0]), checks.host(step.cache.kv_scales[0])
    s0, sl = checks.host(step.swa_start), checks.host(step.swa_len)
    s_gpu = checks.host(step.scores_per_layer[0])
    idx = checks.host(step.idx_per_layer[0])
    L0 = step.layers[0]
    for j, q in enumerate(keep):
        qi = q % wl.q_chunk
        nv = q + 1
        ref = checks.full_index_scores(checks.bf16_to_f64(L0["q_idx"][qi]),
                                       checks.host(L0["w"][qi]).astype(np.float64), ik_c, ik_s, nv)
        checks.check_scores(s_gpu[j, :nv], ref)
        checks.check_topk_exact(idx[j], s_gpu[j, :nv], wl.k)
        checks.check_topk_tolerance(idx[j], ref, wl.k)
        for li in range(len(wl.layers)):
            assert np.array_equal(checks.host(step.idx_per_layer[li])[j], idx[j])   # Reuse layers
            L = step.layers[li]
            sc, ss = checks.swa_rows(checks.host(L["swa_codes"][0]), checks.host(L["swa_scale"][0]).astype(np.float64),
                                     int(s0[q]), int(sl[q]))
            rows = R.gather_rows(kv_c, kv_s, idx[j], sc, ss)
            checks.check_attention(checks.host(step.out_kept[li][j]), checks.host(step.lse_kept[li][j]),
                                   checks.bf16_to_f64(L["q_attn"][qi]), rows)
