"""The CPU baseline's all-cores oracle pass is the oracle itself, split into
independent pieces (layout per source, dispatch per destination rank as a
one-rank problem, combine per token chunk): its results must equal the
single-threaded pass bit for bit."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import bench
import oracle
from combine_get_dispatch_histogram_amd import workloads as wl


@pytest.mark.parametrize("w", [wl.TINY, wl.NormalWorkload("masked", S=3, T=50, H=256, E=48, R=6, K=5, C=7),
                               wl.NORMAL], ids=["tiny", "masked", "normal"])
def test_parallel_pass_equals_single_pass(w):
    inp = wl.normal_inputs(w, 0)
    x = wl.bf16_bits(inp["x"])
    idx = inp["topk_idx"].numpy().copy()
    if w.name == "masked":
        rng = np.random.default_rng(1)
        idx[rng.random(idx.shape) < 0.2] = -1
        idx[rng.random(idx.shape) < 0.05] = w.E + 2            # out of range: ignored like a masked entry
        idx[::4, 1] = idx[::4, 0]                              # duplicated expert
    wts = inp["topk_weights"].numpy()
    lay = oracle.layout(idx, w.S, w.E, w.R)
    d = oracle.dispatch(x, idx, wts, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=w.S, E=w.E, R=w.R,
                        C=w.C)
    y = wl.bf16_bits(wl.expert_outputs(d["num_recv"], w.H, seed=1))
    c = oracle.combine(y, d["recv_topk_weights"], d["send_head"], d["recv_rank_offset"], S=w.S)
    with ThreadPoolExecutor(5) as pool:
        p = bench._oracle_parallel_pass(oracle, w, x, idx, wts, y, pool)
    for k in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank"):
        assert np.array_equal(p[k], lay[k]), k
    for k in ("send_head", "recv_rank_offset", "recv_x", "recv_topk_idx"):
        assert np.array_equal(p[k], d[k]), k
    assert np.array_equal(p["recv_topk_weights"].view(np.uint32), d["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(p["combined_x"], c["combined_x"])
    assert np.array_equal(p["combined_topk_weights"].view(np.uint32), c["combined_topk_weights"].view(np.uint32))
