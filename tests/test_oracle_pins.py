"""Pins of the oracle's layout and accounting against the numbers the pages
print (fixture: tests/golden/page_constants.json)."""
import json
import os

import pytest

from oracle import csa2_ref as R

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_entry_bytes():
    main, idx, tot = R.entry_bytes()
    assert main == G["main_kv_bytes_per_entry"]["value"]
    assert idx == G["indexer_k_bytes_per_entry"]["value"]
    assert tot == G["entry_bytes"]["value"]
    assert main * 8 / R.D_LATENT == G["main_kv_bits_per_channel"]["value"]


def test_layer_schedule():
    sched = R.layer_schedule()
    assert len(sched) == 38
    full = [l for (l, mode, _) in sched if mode == "full"]
    assert full == G["full_layers"]["value"]
    counts = {mode: sum(1 for s in sched if s[1] == mode) for mode in ("full", "reindex", "reuse")}
    assert counts == {k: G["mode_counts"][k] for k in ("full", "reindex", "reuse")}
    eff = sum(1.0 / m for (_, mode, m) in sched if mode == "full")
    assert eff == G["effective_full_layers"]["value"]


def test_890_bytes_per_token():
    assert R.global_kv_bytes_per_token() == G["global_kv_bytes_per_token"]["value"]
    assert R.global_kv_bytes_per_token() * 1e6 == G["global_kv_bytes_at_1M"]["value"]


def test_indexer_mac_model():
    assert R.H_INDEX * R.D_INDEX == G["macs_per_pair"]["value"]
    pool = G["pool_positions"]["value"]
    assert pool == G["pool_positions"]["blocks"] * G["pool_positions"]["block"]
    for n in (4096, 1 << 20, 10 ** 6):
        got = R.indexer_macs_per_decode_token(n, pool)
        assert got == G["decode_indexer_mac_coeff"]["value"] * n + 4 * pool * 4096
        flat = R.indexer_macs_per_decode_token(n, pool, hierarchical=False)
        assert flat == G["decode_indexer_mac_coeff_flat"]["value"] * n
    # 1M context: 10.2 G MAC linear term, 20.5 GFLOPs, about 5.1 at FP4 weight 1/4
    lin = G["decode_indexer_mac_coeff"]["value"] * 1e6
    assert round(lin / 1e9, 1) == 10.2
    assert round(2 * lin / 1e9, 1) == G["decode_indexer_gflops_at_1M"]["value"]
    assert round(2 * lin / 1e9 * 0.25, 1) == G["decode_indexer_weighted_gflops_at_1M"]["value"]
    flat = R.indexer_macs_per_decode_token(10 ** 6, pool, hierarchical=False)
    assert round(2 * flat / 1e9 * 0.25) == G["flat_weighted_gflops_at_1M"]["value"]


def test_prefill_indexer_mac_model():
    # three encoder Full layers (m = 2), N causal raw queries each scoring
    # the visible entries; about 3072 N^2 MACs
    n = 1 << 16
    macs = 0
    for (_, mode, m) in R.layer_schedule():
        if mode == "full" and m == 2:
            visible = sum(((t + 1) // m) for t in range(0, n, 64)) * 64   # sampled sum
            macs += visible * R.H_INDEX * R.D_INDEX
    assert macs / n ** 2 == pytest.approx(G["prefill_indexer_mac_coeff"]["value"], rel=2e-3)
