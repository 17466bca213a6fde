"""The benchmark's byte accounting against the per-token cache sizes the pages print."""
import os

import pytest

from decode_attention_lrkv_amd import bytes_model as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_bytes_per_token.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    return vals


def test_dense_llama31_8b_matches_novakv_card():
    g = _golden()
    b = bm.dense_kv_bytes_per_token(layers=32, n_kv_heads=8, head_dim=128, elem_bytes=2)
    assert b == 131072
    assert round(b / 1000, 2) == g["dense_llama31_8b_kb"]


def test_lowrank_bytes_reproduce_the_card_size_at_mean_rank_142():
    """72.70 KB/token over 32 layers x 8 kv heads x 2 bytes means r_K + r_V averages 142."""
    g = _golden()
    b = bm.lowrank_kv_bytes_per_token(8, [(64, 78)] * 32)
    assert abs(b / 1000 - g["novakv_llama31_8b_kb"]) < 0.01


def test_dense_llama7b_and_kvquant_record():
    g = _golden()
    dense = bm.dense_kv_bytes_per_token(layers=32, n_kv_heads=32, head_dim=128, elem_bytes=2)
    assert dense == g["dense_llama7b_bytes"]
    q = bm.quantized_bytes_per_token(dense, g["kvquant_bits"])
    assert abs(q - g["kvquant_bytes"]) < 1.0


def test_decode_bytes_of_the_batched_workload():
    """Batch 16, 8 kv heads, 32768 tokens, ranks (32, 96) / (48, 112): cache rows dominate."""
    even = bm.decode_bytes(16, 32, 8, 128, 32, 96, 32768)
    odd = bm.decode_bytes(16, 32, 8, 128, 48, 112, 32768)
    assert even == 2 * 16 * 8 * 32768 * 128 + 2 * 8 * 128 * 128 + 2 * 2 * 16 * 32 * 128
    assert odd == 2 * 16 * 8 * 32768 * 160 + 2 * 8 * 128 * 160 + 2 * 2 * 16 * 32 * 128
    # half the dense cache's bytes at r_K + r_V = 128 (the 32-layer step's 56 / 72)
    assert bm.lowrank_kv_bytes_per_token(8, [(56, 72)] * 32) * 2 == bm.dense_kv_bytes_per_token(32, 8, 128)


def test_hybrid_side_tokens_in_bytes():
    full = bm.decode_bytes(1, 32, 8, 128, 64, 64, 131072)
    hyb = bm.decode_bytes(1, 32, 8, 128, 64, 64, 131072, side_tokens=6554)
    assert hyb - full == 8 * 6554 * (2 * 128 * 2 + 4) - 2 * 8 * 6554 * 128


def test_latent_decode_bytes_skip_the_bases():
    """Absorbed projections: the cache rows, r_K-wide queries and r_V-wide outputs; no basis."""
    lat = bm.latent_decode_bytes(16, 32, 8, 48, 112, 32768)
    assert lat == 2 * 16 * 8 * 32768 * 160 + 2 * 16 * 32 * (48 + 112)
    # against the full decode (bases read, d-wide query in and output out)
    full = bm.decode_bytes(16, 32, 8, 128, 48, 112, 32768)
    assert full - lat == 2 * 8 * 128 * 160 + 2 * 2 * 16 * 32 * 128 - 2 * 16 * 32 * 160


def test_oja_bytes_and_flops_of_the_prefill_chunk():
    # 16 x 4096 tokens x 8 heads x 128 dims of bf16 in; float32 basis in and out, bf16 copy out
    assert bm.oja_bytes(16, 4096, 8, 128, 48) == 2 * 16 * 4096 * 8 * 128 + 10 * 8 * 128 * 48
    # Y = X B and X^T Y: 2 d r each; Y^T Y: r^2; times 2 flops per multiply-add
    n = 16 * 4096 * 8
    assert bm.oja_flops(16, 4096, 8, 128, 48) == 2 * n * (2 * 128 * 48 + 48 * 48)
