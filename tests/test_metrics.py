"""Workload arithmetic against the figures the pages print (tests/golden/metric_examples.json)."""
import json
import os

from exact_tiled_attention_flash_amd import metrics

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "metric_examples.json")))


def test_causal_flops_matches_page_snippet():
    assert metrics.fwd_flops(8, 16, 2048, 64, causal=True) == GOLD["causal_fwd_flops_b8h16t2048d64"]["value"]
    assert metrics.fwd_flops(8, 16, 2048, 64, causal=False) == 2 * GOLD["causal_fwd_flops_b8h16t2048d64"]["value"]


def test_score_matrix_bytes():
    assert metrics.score_matrix_bytes(8, 16, 2048, 2) == GOLD["score_matrix_bytes_b8h16t2048_bf16"]["value"]
    assert metrics.score_matrix_bytes(1, 1, 8192, 2) == GOLD["score_matrix_bytes_per_head_t8192_bf16"]["value"]


def test_arithmetic_intensity_example():
    ai = metrics.fwd_flops(1, 8, 1024, 64, False) / metrics.fwd_bytes(1, 8, 1024, 64, 2, with_lse=False)
    assert ai > GOLD["arith_intensity_b1h8t1024d64_fp16_min"]["value"]
    assert ai == 1024 / 2  # T/2 exactly


def test_headline_numbers():
    # causal bf16, B=4 H=16 T=4096 D=128
    assert metrics.fwd_flops(4, 16, 4096, 128, True) == 274877906944
    assert metrics.fwd_bytes(4, 16, 4096, 128, 2) == 268435456 + 1048576
