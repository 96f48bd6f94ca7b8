"""Benchmark of one decode step of the CSA2 global branch on one MI355X.

Default workload: hierarchical decoder decode at 1M context (batch 4,
N = 2^20 FP4 entries per sequence): the Full layer scans all entries,
builds the 2048 x 8 block pool and its top-512 and attends; 4 Reindex
layers rescore the pool with their own queries, take their top-512 and
attend.  A step is that whole 5-layer pass; tokens/s = batch / step time.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line with the metric, a roofline entry for the dominant
kernel (the Full layer's index scan, timed with HIP events on its stream
inside the timed region) and the fp64 oracle's speed on a bounded sample
of the same workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_sparse_csa2_amd import synth  # noqa: E402
from long_context_sparse_csa2_amd.pipeline import Step  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD datasheet
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix peak, AMD datasheet
MFMA_FP4_PEAK_TFLOPS = 10100.0 # MI355X dense fp4 matrix peak, AMD datasheet
SCAN_BYTES_PER_ENTRY = 68      # MXFP4 indexer K: 64 B codes + 4 B E8M0 scales
SCAN_FLOPS_PER_ENTRY = 2 * 32 * 128   # 32 heads x 128 dims multiply-adds per (query, entry)
METRIC = "decode tokens/s at 1M ctx (indexer+top-512+FP4 sparse attn); % of roofline"
PREFILL_METRIC = "prefill raw tokens/s (causal indexer+top-512+FP4 sparse attn); % of roofline"


def step_bytes(wl):
    """Algorithmic HBM bytes of one decode step: indexer K of every scanned
    entry, 288 B per gathered main-KV row, 516 B per SWA row, queries and
    outputs.  None for a prefill chunk, whose queries share one sequence
    (its rows are re-read from cache, not HBM)."""
    if wl.prefill:
        return None
    Q = wl.Q
    n_attend = len(wl.layers)
    b = Q * wl.N * SCAN_BYTES_PER_ENTRY
    b += sum(Q * wl.n_blocks * wl.block * SCAN_BYTES_PER_ENTRY for m in wl.layers if m == "reindex")
    b += n_attend * Q * (wl.k * 288 + wl.swa * 516 + 64 * 512 * 2 + 64 * 512 * 4)
    return b


def scan_traffic(cfg, fp4q=False):
    """HBM bytes (read + written) per scan launch from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none or
    the scan kernel's source has changed since the counters were taken."""
    import hashlib
    import re
    kind = "index_score_fp4q" if fp4q else "index_score"
    f = os.path.join(ROOT, "profiles", f"{kind}_{cfg}_hbm_traffic.md")
    if not os.path.exists(f):
        return None
    txt = open(f).read()
    m = {k: re.search(rf"^{k}: (\S+)$", txt, re.M) for k in
         ("source_sha256", "fetch_bytes_per_launch", "write_bytes_per_launch")}
    if not all(m.values()):
        return None
    src = os.path.join(ROOT, "long_context_sparse_csa2_amd", "csrc", "score.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m["source_sha256"].group(1):
        return None
    return int(m["fetch_bytes_per_launch"].group(1)) + int(m["write_bytes_per_launch"].group(1))


def scan_roofline(wl, step, scan_us):
    """Roofline entry of the Full-layer scan.  Decode scans stream every
    visible entry's 68 B of indexer K once per query (HBM-bound); a prefill
    chunk scores thousands of queries against the same few thousand entries,
    which stay in cache, so its bound is the MFMA work instead (bf16 for the
    bf16 query, fp4 for the MXFP4 query).  The bound is whichever takes
    longer at its datasheet peak."""
    n_vis = step.n_vis.cpu().numpy()
    seqs = step.q_seq.cpu().numpy()
    pairs = int(n_vis.sum())
    uniq = sum(int(n_vis[seqs == b].max()) for b in set(seqs.tolist()))  # entries read at least once
    hbm_bytes = (pairs if len(seqs) == len(set(seqs.tolist())) else uniq) * SCAN_BYTES_PER_ENTRY
    flops = pairs * SCAN_FLOPS_PER_ENTRY
    t_hbm = hbm_bytes / (HBM_PEAK_GBS * 1e9)
    peak = MFMA_FP4_PEAK_TFLOPS if step.fp4q else MFMA_BF16_PEAK_TFLOPS
    t_mfma = flops / (peak * 1e12)
    base = {"kernel": "k_index_score (Full-layer scan)", "avg_launch_us": round(scan_us, 2)}
    if t_hbm >= t_mfma:
        achieved = hbm_bytes / (scan_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": scan_traffic(wl.name, step.fp4q),
                "bytes_per_launch": hbm_bytes, **base}
    achieved = flops / (scan_us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "mfma_dtype": "fp4" if step.fp4q else "bf16",
            "traffic": scan_traffic(wl.name, step.fp4q), "flops_per_launch": flops, **base}


def measure_peaks(dev, read_bytes=2 << 30, mfma_iters=4000, reps=5):
    """The device's practical ceilings, timed here with HIP events around
    single launches (median of reps): a streaming read of read_bytes by a
    grid-stride kernel (csa2_peak_read) and dense bf16 32x32x16 MFMA chains
    (csa2_peak_mfma).  Reported beside the datasheet peaks, which the
    roofline fractions use."""
    from long_context_sparse_csa2_amd import lib
    L = lib()
    st = torch.cuda.current_stream().cuda_stream
    buf = torch.ones(read_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    fsink = torch.zeros(1024, dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(); fn(); e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_read = timed(lambda: L.csa2_peak_read(buf.data_ptr(), read_bytes, sink.data_ptr(), st))
    flops = [0.0]

    def mf():
        flops[0] = L.csa2_peak_mfma(mfma_iters, fsink.data_ptr(), st)
    t_mfma = timed(mf)
    del buf
    return {"hbm_read_GBs": round(read_bytes / t_read / 1e9, 1),
            "bf16_mfma_TFLOPs": round(flops[0] / t_mfma / 1e12, 1),
            "datasheet_hbm_GBs": HBM_PEAK_GBS, "datasheet_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
            "method": f"csa2_peak_read over {read_bytes >> 20} MiB and csa2_peak_mfma "
                      f"({mfma_iters} iterations of 4 bf16 32x32x16 MFMA chains in 4096 waves), "
                      f"HIP events around single launches, median of {reps}"}


def time_scan_cold(step, dev, reps=10, sweep_bytes=512 << 20):
    """The Full-layer scan timed right after a streaming read of sweep_bytes
    of other memory (which evicts what the 256 MB memory-side cache held of
    the scan's bytes from the previous step): HIP events on the current
    stream, median of reps, microseconds."""
    from long_context_sparse_csa2_amd import lib
    L = lib()
    st = torch.cuda.current_stream().cuda_stream
    buf = torch.ones(sweep_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    op = step.ops()[step.scan_index()]
    ts = []
    for _ in range(reps):
        L.csa2_peak_read(buf.data_ptr(), sweep_bytes, sink.data_ptr(), st)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(); op.fn(); e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    del buf
    return float(np.median(ts))


def time_append(wl, dev, calls=64):
    """Decode-time append (csa2_decode_append) of one token per sequence for
    the workload's batch and m, into a fresh state and a cache with room for
    the appended entries: `calls` back-to-back calls captured in one HIP
    graph, replayed between HIP events on the current stream.  Returns
    microseconds per call."""
    from long_context_sparse_csa2_amd import Cache, State, csa2_decode_append
    B, m = wl.B, wl.m
    cache = Cache(B, calls // m + 1, dev)
    st = State(B, m, wl.swa, dev)
    g = torch.Generator(device=dev).manual_seed(5)
    h = torch.randn(calls, B, 512, device=dev, generator=g).to(torch.bfloat16)
    z = torch.randn(calls, B, 512, device=dev, generator=g).to(torch.bfloat16) if m > 1 else None
    sw = torch.randn(calls, B, 512, device=dev, generator=g).to(torch.bfloat16)
    w_ik = wl.w_ik(dev)
    n_vis = torch.empty(B, dtype=torch.int64, device=dev)
    s0 = torch.empty(B, dtype=torch.int64, device=dev)
    sl = torch.empty(B, dtype=torch.int32, device=dev)
    def run():
        for i in range(calls):
            csa2_decode_append(h[i], z[i] if z is not None else None, sw[i], w_ik, cache, st,
                               n_vis, s0, sl)
    run()                                     # eager pass (loads the kernels)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    st.n_tok.zero_()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def time_attend_rope(step, dev, calls=20):
    """The fused RoPE - attention - inverse RoPE - bf16 cast
    (csa2_sparse_attend_rope, 64 rotated channels, theta 10000) on the step's
    first layer (its queries, selection and SWA windows), next to the plain
    csa2_sparse_attend on the same inputs: `calls` launches of each captured
    in a HIP graph and replayed between HIP events.  Returns microseconds per
    call (rope, plain)."""
    from long_context_sparse_csa2_amd import csa2_sparse_attend, csa2_sparse_attend_rope
    wl = step.wl
    L = step.layers[0]
    Q = wl.Q if not step.chunks or len(step.chunks) == 1 else step.chunks[0][1]
    rows = slice(0, Q)
    pos = (torch.arange(Q, dtype=torch.int64, device=dev) * 7919 + (1 << 20) - 1)
    out_b = torch.empty(Q, 64, 512, dtype=torch.bfloat16, device=dev)
    out_f = torch.empty(Q, 64, 512, dtype=torch.float32, device=dev)
    args = (L["q_attn"][rows], step.q_seq[rows], step.cache, step.idx[:Q], L["swa_codes"],
            L["swa_scale"], step.swa_start[rows], step.swa_len[rows])
    res = []
    for fn in (lambda: csa2_sparse_attend_rope(*args, pos, 64, 10000.0, out_b, None, step.ws_attend),
               lambda: csa2_sparse_attend(*args, out_f, None, step.ws_attend)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(calls):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(); g.replay(); e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / calls)
    return res


def blas_threads():
    """Threads the oracle's numpy BLAS runs on (its matmuls; the elementwise
    steps run on one)."""
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])


def host_cpus():
    return {"host_cpus": os.cpu_count(), "cpus_in_affinity": len(os.sched_getaffinity(0))}


def cpu_baseline_prefill(wl, step, seconds_target=15.0):
    """The fp64 oracle on a sample of a prefill's queries, spread over the
    causal range: per query, its entry compressed from its m raw tokens, then
    every layer (scores over its visible entries, top-512, attention with its
    SWA window).  One query stands for m raw
    tokens, so tokens/s = m x queries / s (the work grows with the position,
    and the sample is spread evenly, so its mean matches the whole run's)."""
    from oracle import csa2_ref as R
    ik_c = step.cache.ik_codes[0].cpu().numpy()
    ik_s = step.cache.ik_scales[0].cpu().numpy()
    kv_c = step.cache.kv_codes[0].cpu().numpy()
    kv_s = step.cache.kv_scales[0].cpu().numpy()
    n_vis = step.n_vis.cpu().numpy()
    s0, sl = step.swa_start.cpu().numpy(), step.swa_len.cpu().numpy()
    khat = R.dequant_mxfp4(ik_c, ik_s)
    scores = R.index_scores_fp4q if step.fp4q else R.index_scores
    order = np.random.default_rng(0).permutation(wl.Q)     # spread over the causal range
    m = wl.m
    w_ik = step.w_ik.float().cpu().numpy().astype(np.float64)
    done, t_total = 0, 0.0
    while t_total < seconds_target and done < len(order):
        q = int(order[done])
        qi = q % wl.q_chunk if step.reuse else q        # row of the per-layer inputs
        hq = step.h[0, q * m:(q + 1) * m].float().cpu().numpy().astype(np.float64)
        zq = None if step.z is None else step.z[0, q * m:(q + 1) * m].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        R.build_entries(hq, zq, m, w_ik)          # the query's own entry from its m raw tokens
        idx = None
        for li, mode in enumerate(wl.layers):
            L = step.layers[li]
            if mode == "full":
                s = scores(L["q_idx"][qi].float().cpu().numpy().astype(np.float64),
                           L["w"][qi].cpu().numpy().astype(np.float64), khat[:int(n_vis[q])])
                idx = R.topk(s, wl.k)
            sc = L["swa_codes"][0, int(s0[q]):int(s0[q]) + int(sl[q])].cpu().numpy()
            ss = L["swa_scale"][0, int(s0[q]):int(s0[q]) + int(sl[q])].cpu().numpy().astype(np.float64)
            rows = R.gather_rows(kv_c, kv_s, idx, sc, ss)
            R.attend(L["q_attn"][qi].float().cpu().numpy().astype(np.float64), rows)
        t_total += time.perf_counter() - t0
        done += 1
    threads = blas_threads()
    return {"value": wl.m * done / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            **host_cpus(),
            "sample": f"{done} of {wl.Q} queries drawn evenly over the causal range, each its "
                      f"entry's compression and all {len(wl.layers)} layers, {t_total:.1f} s; m = {wl.m} raw tokens per "
                      f"query; numpy fp64 (BLAS matmul on {threads} threads)"}


def cpu_baseline(wl, step, seconds_target=15.0):
    """The fp64 oracle, as it stands, on one sequence of the workload: the
    whole step (Full scan, pool, top-512, attention, every Reindex layer).
    Returns tokens/s for that one-sequence sample."""
    from oracle import csa2_ref as R
    if wl.prefill:
        return cpu_baseline_prefill(wl, step, seconds_target)

    b = 0
    kv_c = step.cache.kv_codes[b].cpu().numpy()
    kv_s = step.cache.kv_scales[b].cpu().numpy()
    ik_c = step.cache.ik_codes[b].cpu().numpy()
    ik_s = step.cache.ik_scales[b].cpu().numpy()
    layers = []
    for li in range(len(wl.layers)):
        L = step.layers[li]
        layers.append(dict(q_idx=L["q_idx"][b].float().cpu().numpy().astype(np.float64),
                           w=L["w"][b].cpu().numpy().astype(np.float64),
                           q_attn=L["q_attn"][b].float().cpu().numpy().astype(np.float64),
                           swa_c=L["swa_codes"][b].cpu().numpy(),
                           swa_s=L["swa_scale"][b].cpu().numpy().astype(np.float64)))
    scores = R.index_scores_fp4q if step.fp4q else R.index_scores
    runs, t_total = 0, 0.0
    while t_total < seconds_target and runs < 5:
        t0 = time.perf_counter()
        khat = R.dequant_mxfp4(ik_c, ik_s)
        pool = None
        for li, mode in enumerate(wl.layers):
            L = layers[li]
            if mode == "full":
                s = scores(L["q_idx"], L["w"], khat)
                if wl.hierarchical:
                    pool = R.block_pool(s, wl.block, wl.n_blocks)
                idx = R.topk(s, wl.k)
            elif mode == "reindex":
                s = scores(L["q_idx"], L["w"], khat[pool])
                idx = R.topk(s, wl.k, pool)
            rows = R.gather_rows(kv_c, kv_s, idx, L["swa_c"], L["swa_s"])
            R.attend(L["q_attn"], rows)
        t_total += time.perf_counter() - t0
        runs += 1
    threads = blas_threads()
    return {"value": runs / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            **host_cpus(),
            "sample": f"one of {wl.B} sequences, whole {len(wl.layers)}-layer step, "
                      f"{runs} run(s) in {t_total:.1f} s; numpy fp64 (BLAS matmul on "
                      f"{threads} threads, elementwise steps on 1)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--indexer-q", default="bf16", choices=["bf16", "mxfp4"],
                    help="indexer query format: bf16 as given, or quantised to MXFP4 in the "
                         "scan (csa2_index_score_fp4q)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python "
                    "instead of replaying the step's HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path would shard by sequence across GPUs, which is not implemented",
              file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    wl = synth.WORKLOADS[args.config]
    print(f"[bench] building {wl.name} ({wl.note}) cache on {dev}", file=sys.stderr, flush=True)
    step = Step(wl, dev, fp4q=args.indexer_q == "mxfp4")
    torch.cuda.synchronize()
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # eager pass with per-call events (breakdown of the step)
    events = {}
    for _ in range(3):
        step.run(events=events)
    torch.cuda.synchronize()
    per_call = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) * 1e3 for k, v in events.items()}
    calls = {k: len(v) // 3 for k, v in events.items()}

    # Timed region: K steps.  Graph mode replays the whole step as one HIP
    # graph (timing events cannot be recorded inside a graph here, and a
    # timing event between launches costs the step several microseconds);
    # the Full-layer scan's duration then comes from K further steps right
    # after it, each launched as [scan between HIP events on its stream] +
    # [the rest of the step as a graph].  A chunked prefill launches eagerly
    # (its calls run for milliseconds) and times every chunk's scan inside
    # the timed region; so does --eager.
    chunked = len(step.chunks) > 1
    graphs = None if (args.eager or chunked) else step.capture(split_first=True)
    whole = None if graphs is None else step.capture(split_first=False)[0]
    ops = step.ops()                      # built before any timed loop: the host only enqueues
    n_scans = sum(op.name == "index_score_full" for op in ops)
    i_scan = step.scan_index()
    g_pre = graphs[0] if graphs and i_scan > 0 else None     # calls before the scan (compressor)

    def scan_pass():
        """K steps with the Full-layer scans between HIP events; returns
        (ms per step, scan microseconds per step)."""
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(n_scans)] for _ in range(args.steps)]
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a0.record()
        for si in range(args.steps):
            pairs = evs[si]
            if graphs:
                e0, e1 = pairs[0]
                if g_pre is not None:
                    g_pre.replay()
                e0.record(); ops[i_scan].fn(); e1.record(); graphs[-1].replay()
            else:
                j = 0
                for op in ops:
                    if op.name == "index_score_full":
                        e0, e1 = pairs[j]
                        j += 1
                        e0.record(); op.fn(); e1.record()
                    else:
                        op.fn()
        a1.record()
        torch.cuda.synchronize()
        sus = float(np.mean([sum(x.elapsed_time(y) for x, y in st) for st in evs])) * 1e3
        return a0.elapsed_time(a1) / args.steps, sus

    if whole is not None:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            whole.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        ms_split, scan_us = scan_pass()
    else:
        ms, scan_us = scan_pass()
        ms_split = None
    print(f"[bench] {ms:.3f} ms/step ({'eager' if graphs is None else 'one graph'}); "
          + (f"{ms_split:.3f} ms/step with the scan between events; " if ms_split else "")
          + f"scan {scan_us:.1f} us; eager per call (us): "
          + ", ".join(f"{k}={v:.1f}x{calls[k]}" for k, v in per_call.items()), file=sys.stderr,
          flush=True)

    roofline = scan_roofline(wl, step, scan_us)
    if not chunked:
        # the same scan right after a 512 MiB read sweep of other memory
        roofline["avg_launch_us_after_read_sweep"] = round(time_scan_cold(step, dev), 2)
    peaks = measure_peaks(dev)
    step_b = step_bytes(wl)
    out = {
        "metric": PREFILL_METRIC if wl.prefill else METRIC,
        "value": round((wl.T if wl.prefill else wl.B) / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "batch": wl.B, "entries": wl.N,
                   "raw_tokens": wl.T, "m": wl.m, "layers": wl.layers, "top_k": wl.k,
                   "pool_blocks": wl.n_blocks if wl.hierarchical else 0, "swa": wl.swa,
                   "indexer_q": args.indexer_q, "query_chunk": wl.q_chunk if wl.prefill else 0},
        "roofline": roofline,
        "step_roofline": None if step_b is None else {
            "bytes": step_b, "us_at_peak": round(step_b / (HBM_PEAK_GBS * 1e3), 2),
            "frac": round(step_b / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4)},
        "peaks_measured": peaks,
        "launch": "eager" if graphs is None else "the step replayed as one hip graph",
        "scan_timing": ("HIP events around each Full-layer scan inside the timed region"
                        if graphs is None else
                        f"HIP events around the scan in {args.steps} further steps launched as "
                        "scan + the rest of the step as a graph, right after the timed region"),
        "ms_per_step_scan_between_events": None if ms_split is None else round(ms_split, 4),
        "per_call_us_eager": {k: round(v, 2) for k, v in per_call.items()},
        "calls_per_step": calls,
    }
    rope_us, plain_us = time_attend_rope(step, dev)
    out["attend_rope"] = {"us_per_call": round(rope_us, 2), "plain_us_per_call": round(plain_us, 2),
                          "queries": step.chunks[0][1], "rope_dims": 64,
                          "note": "csa2_sparse_attend_rope (bf16 out) vs csa2_sparse_attend "
                                  "(fp32 out) on the first layer's inputs; not part of the step"}
    if not wl.prefill:
        out["decode_append"] = {"us_per_call": round(time_append(wl, dev), 2), "batch": wl.B,
                                "m": wl.m, "swa_window": wl.swa,
                                "note": "csa2_decode_append, one HIP graph of 64 calls; not part of the step"}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, step)
        if wl.name in ("c0", "c1"):
            # the same oracle on one host thread
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                one = cpu_baseline(wl, step)
            out["cpu_baseline_1thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
