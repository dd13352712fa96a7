"""Pins for the oracle's KV byte model (CPU only), against numbers the pages print."""
import json
import os

import pytest

from oracle import byte_model as bm

G = os.path.join(os.path.dirname(__file__), "golden")


def test_pd_page_worked_kv_sizes():
    g = json.load(open(os.path.join(G, "pd_page_kv_bytes.json")))
    per_tok = bm.kv_bytes_per_token(g["kv_heads"], g["head_dim"], g["dtype"])
    assert per_tok == g["bytes_per_token_per_layer"]
    per_layer = bm.kv_cache_bytes(1, g["kv_heads"], g["head_dim"], g["tokens"], g["dtype"])
    assert per_layer == g["bytes_per_layer_MB"] * 2 ** 20
    total = bm.kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["tokens"], g["dtype"])
    assert total == g["total_MB"] * 2 ** 20
    t = g["transfer_times_ms_for_256MB"]
    assert 256e6 / 900e9 * 1e3 == pytest.approx(t["nvlink4_900GBps"], abs=0.005)
    assert 256e6 / (400e9 / 8) * 1e3 == pytest.approx(t["gdr_400Gbps"], abs=0.05)


def test_nanopd_cost_model_ratios_need_qwen3_8b_kv_bytes():
    g = json.load(open(os.path.join(G, "nanopd_cost_model.json")))
    per_tok = bm.kv_bytes_per_token(8, 128, "bf16", layers=36)      # Qwen3-8B: 36 layers
    assert per_tok == 147456
    for hw, want in g["gamma_over_transfer_rate"].items():
        rate_ms = per_tok / (g["bandwidth_GBps"][hw] * 1e9) * 1e3   # ms per token moved
        got = g["gamma_ms_per_token"][hw] / rate_ms
        assert got == pytest.approx(want, rel=0.005), hw


def test_prefill_flops_count_unmasked_pairs():
    # prefix 0, chunk 3: rows see 1, 2, 3 keys -> 6 pairs
    assert bm.prefill_chunk_flops([0], [3], 1, 1) == 4 * 6
    assert bm.prefill_chunk_flops([10], [2], 32, 128) == 4 * 128 * 32 * (11 + 12)


def test_decode_bytes():
    assert bm.decode_kv_bytes([17, 33, 64, 100], 2, 64, "f32") == 214 * 1024
