"""Byte and FLOP accounting against the counts the pages print (CPU only)."""
import json
import os

import pytest

from exact_scaled_dot_sdpa_amd import accounting as A

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_byte_counts.json")))
UNIT = {"MiB": 2 ** 20, "GiB": 2 ** 30}


@pytest.mark.parametrize("case", GOLD["score_matrix"], ids=lambda c: "n%d_h%d" % (c["n"], c["heads"]))
def test_score_matrix_bytes(case):
    assert A.score_matrix_bytes(case["n"], case["elem_bytes"], case["heads"]) == case["value"] * UNIT[case["unit"]]


@pytest.mark.parametrize("case", GOLD["kv_cache"], ids=lambda c: "L%d_n%d_b%d" % (c["layers"], c["n"], c["batch"]))
def test_kv_cache_bytes(case):
    got = A.kv_cache_bytes(case["layers"], case["n"], case["h_kv"], case["d_h"], case["elem_bytes"], case["batch"])
    assert got == case["value"] * UNIT[case["unit"]]


@pytest.mark.parametrize("case", GOLD["pair_counts"], ids=lambda c: "n%d" % c["n"])
def test_pair_counts(case):
    got = A.visible_pairs(case["n"], case["n"], False)
    if "pairs" in case:
        assert got == case["pairs"]
    else:
        assert abs(got - case["pairs_approx"]) <= case["rel_tol"] * case["pairs_approx"]


def test_causal_pairs():
    # square causal: N(N+1)/2; bottom-right alignment for Nq < Nk
    assert A.visible_pairs(8192, 8192, True) == 8192 * 8193 // 2
    assert A.visible_pairs(1, 100, True) == 100
    assert A.visible_pairs(3, 5, True) == 3 + 4 + 5
    assert A.visible_pairs(0, 5, True) == 0


def test_workload_figures():
    # the figures quoted for the GQA prefill and the decode workloads
    assert A.prefill_flops(1, 64, 8192, 8192, 128, True) == 1_099_645_845_504
    assert A.prefill_bytes(1, 64, 8, 8192, 8192, 128, "bf16") == 304_087_040
    sl = [512, 4096]
    assert A.decode_bytes(sl, 32, 8, 128, "bf16") == 4096 * sum(sl) + 2 * 2 * 32 * 128 * 2 + 4 * 2 + 4 * 2 * 32
    assert A.decode_flops(sl, 32, 128) == 4 * 128 * 32 * sum(sl)


def test_bwd_flops_is_two_and_a_half_forward():
    for (Nq, Nk, causal) in ((100, 100, True), (64, 333, True), (50, 70, False)):
        assert 2 * A.bwd_flops(2, 4, Nq, Nk, 64, causal) == 5 * A.prefill_flops(2, 4, Nq, Nk, 64, causal)
