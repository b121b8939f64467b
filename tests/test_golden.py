"""The oracle reproduces the stored fixtures: the pages' own constants, and the
tiny-workload digests written by tests/golden/make_golden.py (a regression
guard on the oracle's arithmetic)."""
import json
import os

import numpy as np

import brute
from golden.make_golden import tiny

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_pages_constants(orc):
    g = _load("pages_constants.json")
    assert orc.ll_msg_bytes(7168, True) == g["ll_msg_bytes_fp8_h7168"]["value"]
    assert orc.ll_msg_bytes(7168, False) == g["ll_msg_bytes_bf16_h7168"]["value"]
    e = g["expected_ranks_per_token_normal"]
    assert abs(brute.expected_groups_hit(256, 8, 8) - e["value"]) < e["tol"]
    e = g["expected_ranks_per_token_large"]
    assert abs(brute.expected_groups_hit(256, 8, 64) - e["value"]) < e["tol"]
    # rank r belongs to RDMA group r // 8: 64 ranks -> 8 groups of the layout
    idx = np.array([[0, 4 * 9, 4 * 63]], np.int64)            # experts on ranks 0, 9, 63 (E = 256, R = 64)
    lay = orc.layout(idx, 1, 256, 64)
    assert lay["num_tokens_per_rdma_rank"].tolist() == [[1, 1, 0, 0, 0, 0, 0, 1]]
    assert g["ranks_per_rdma_group"]["value"] == 8


def test_tiny_digests(orc):
    assert tiny() == _load("tiny_seed0.json")
