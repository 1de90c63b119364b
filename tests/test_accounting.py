"""CPU pins for the benchmark's work accounting.

The closed-form visible-pair count is checked against the oracle's
enumeration of the mask predicate, and the byte/size accounting against the
sizes the pages print.
"""
import json
import os

import pytest

from online_softmax_fa2_amd import accounting as acc
from online_softmax_fa2_amd.inputs import WORKLOADS
from oracle import visible_count

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


@pytest.mark.parametrize("N,kv,causal,window", [
    (1, None, False, 0), (1000, None, False, 0), (1000, None, True, 0), (777, 500, True, 33), (640, 600, False, 100),
    (300, 0, True, 5), (2048, None, True, 0), (513, 257, False, 1000), (400, None, True, 1),
])
def test_visible_pairs_matches_enumeration(N, kv, causal, window):
    assert acc.visible_pairs(N, kv, causal, window) == visible_count(N, N if kv is None else kv, causal, window)


def test_headline_workload_flops():
    w = WORKLOADS["attn_bf16_causal_w1024_pad512_b1h64_n8192_d128"]
    pairs = visible_count(w["N"], w["kv_len"][0], w["causal"], w["window"])
    assert acc.attn_flops(w["B"], w["H"], w["N"], w["d"], w["causal"], w["window"], w["kv_len"]) == 4 * 128 * 64 * pairs
    w3 = WORKLOADS["attn_bf16_causal_b4h32_n2048_d128"]
    assert acc.attn_flops(4, 32, 2048, 128, True, 0) == 4 * 128 * 128 * 2048 * 2049 // 2


def test_score_matrix_size_matches_page():
    f = FACTS["score_matrix_bytes_per_head_8k_bf16"]
    per_head = 8192 * 8192 * 2
    assert per_head == f["value_mib"] * 2 ** 20
    assert per_head * f["heads"] == f["per_layer_gib"] * 2 ** 30


def test_tile_state_sizes_match_page():
    f = FACTS["tile_state_sizes"]
    assert f["Br"] * f["d"] * 4 == f["acc_kib"] * 1024
    assert 2 * f["Br"] * 4 == f["m_l_kib"] * 1024
    assert f["Br"] * f["Bc"] * 4 == f["score_tile_kib"] * 1024
    assert 8192 // f["Bc"] == f["key_blocks_per_tile_at_8192"]
    assert f["Br"] * f["d"] == f["fa2_divides_per_tile"]


def test_nxn_sizes_match_page():
    f = FACTS["nxn_fp16_gib_per_head"]
    for n, gib in zip(f["N"], f["gib"]):
        assert round(n * n * 2 / 2 ** 30, 3) == pytest.approx(gib, abs=5e-4)


def test_byte_accounting():
    assert acc.decode_bytes(1, 32, 131072, 128) == 2 ** 31
    assert acc.softmax_bytes(4096, 4000) == 131_072_000
    assert acc.topk_bytes(1024, 25000, 5) == 102_400_000 + 1024 * 40
