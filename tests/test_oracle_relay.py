"""Pins for the oracle's two-level relay (dispatch through one RDMA buffer per
group of 8 ranks, forwarding to the group's ranks, and the two-level
combine): an independent brute force, the flat dispatch it must reproduce on
the receive side, the layout's per-RDMA-rank counts, the identity round trip
and the exact weight reduction."""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_histogram_amd import workloads as wl
from tests import brute

SHAPES = [
    # name, S, T, H, E, R, K, C
    ("r16", 4, 24, 256, 32, 16, 4, 3),
    ("r24", 3, 30, 128, 48, 24, 5, 4),
    ("r64", 2, 40, 128, 256, 64, 8, 5),
    ("r8", 3, 20, 128, 16, 8, 3, 2),          # one group
    ("empty", 2, 0, 128, 32, 16, 4, 3),
]


def _inputs(S, T, H, E, R, K, C, seed, masked=False):
    w = wl.NormalWorkload("relay", S=S, T=T, H=H, E=E, R=R, K=K, C=C)
    inp = wl.normal_inputs(w, seed)
    idx = inp["topk_idx"].numpy().copy()
    if masked and idx.size:
        rng = np.random.default_rng(seed)
        idx[rng.random(idx.shape) < 0.2] = -1
        if K > 1:
            d = rng.random(idx.shape[0]) < 0.2
            idx[d, 1] = idx[d, 0]
    return w, wl.bf16_bits(inp["x"]), idx, inp["topk_weights"].numpy()


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("masked", [False, True], ids=["plain", "masked-dup"])
def test_relay_dispatch_matches_brute_and_flat(shape, masked):
    name, S, T, H, E, R, K, C = shape
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 3, masked)
    lay = oracle.layout(idx, S, E, R)
    itr = lay["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C)
    G = R // 8
    rows, srh, nvl = brute.relay_plan(itr, S)
    # first hop: group buffers and heads
    assert np.array_equal(r["send_rdma_head"], srh)
    roff = r["recv_rdma_offset"]
    assert np.array_equal(np.diff(roff), [len(rows[g]) for g in range(G)])
    for g in range(G):
        for i, n in enumerate(rows[g]):
            q = roff[g] + i
            assert r["rdma_src_idx"][q] == n
            assert np.array_equal(r["rdma_x"][q], x[n])
            assert list(r["send_nvl_head"][q]) == nvl[(g, i)]
    # rdma prefix matrices = the O2 definitions over group membership
    grp = itr.reshape(itr.shape[0], G, 8).any(axis=2).astype(np.uint8)
    _, cpm, rpm, rcpm = brute.dispatch_plan(grp, S, C)
    assert np.array_equal(r["rdma_channel_prefix_matrix"], cpm)
    assert np.array_equal(r["rdma_rank_prefix_matrix"], rpm)
    assert np.array_equal(r["recv_rdma_channel_prefix_matrix"], rcpm)
    # the layout's per-RDMA-rank counts are the per-source group row counts
    if R > 8:
        per_src = np.diff(np.vstack([np.zeros((1, G), np.int64), r["rdma_rank_prefix_matrix"]]), axis=0)
        assert np.array_equal(per_src, lay["num_tokens_per_rdma_rank"])
    # second hop: the receive side is the flat dispatch's
    d = oracle.dispatch(x, idx, wts, itr, lay["num_tokens_per_expert"], S=S, E=E, R=R, C=C)
    for k in ("recv_x", "recv_src_idx", "recv_topk_idx", "recv_rank_offset"):
        assert np.array_equal(r[k], d[k]), k
    assert np.array_equal(r["recv_topk_weights"].view(np.uint32), d["recv_topk_weights"].view(np.uint32))


@pytest.mark.parametrize("round_scale", [False, True])
def test_relay_fp8_cast_once_before_first_hop(round_scale):
    S, T, H, E, R, K, C = 2, 16, 256, 32, 16, 4, 2
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 5)
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C, x_kind=oracle.X_BF16_CAST_FP8,
                              round_scale=round_scale)
    n = r["num_rdma_recv"]
    for q in range(n):
        src = r["rdma_src_idx"][q]
        codes, scales, _ = brute.fp8_quantize_row(x[src], round_scale)
        assert list(r["rdma_x"][q]) == codes
        assert np.array_equal(r["rdma_x_scales"][q], np.array(scales, np.float32))
    # the forwarded rows are byte copies of the group rows: equal to the flat FP8-cast dispatch
    lay = oracle.layout(idx, S, E, R)
    d = oracle.dispatch(x, idx, wts, itr, lay["num_tokens_per_expert"], S=S, E=E, R=R, C=C,
                        x_kind=oracle.X_BF16_CAST_FP8, round_scale=round_scale)
    assert np.array_equal(r["recv_x"], d["recv_x"])
    assert np.array_equal(r["recv_x_scales"].view(np.uint32), d["recv_x_scales"].view(np.uint32))


@pytest.mark.parametrize("shape", SHAPES[:3], ids=[s[0] for s in SHAPES[:3]])
@pytest.mark.parametrize("partial_f32", [False, True], ids=["bf16-partials", "fp32-partials"])
def test_relay_combine_matches_brute(shape, partial_f32):
    name, S, T, H, E, R, K, C = shape
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 7, masked=True)
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C)
    y = wl.bf16_bits(wl.expert_outputs(r["num_recv"], H, seed=9))
    c = oracle.relay_combine(y, r["recv_topk_weights"], r["recv_rank_offset"], r["recv_rdma_offset"],
                             r["send_nvl_head"], r["send_rdma_head"], S=S, partial_f32=partial_f32, want_f32=True)
    rows, srh, nvl = brute.relay_plan(itr, S)
    out, partial = brute.relay_combine(y, r["recv_rank_offset"], rows, srh, nvl, S, partial_f32=partial_f32)
    assert np.array_equal(c["combined_x"], out)
    roff = r["recv_rdma_offset"]
    for (g, i), p in partial.items():
        got = c["rdma_y"][roff[g] + i]
        assert np.array_equal(got.view(np.uint32) if partial_f32 else got, p.view(np.uint32) if partial_f32 else p)
    # the reported fp32 sums are the values the output rounds (torch's cast)
    assert np.array_equal(brute.bf16_round_lib(c["combined_f32"]).reshape(out.shape), out)


def test_relay_combine_fp32_partials_error_bound():
    """With fp32 partials the two-level result is one fp32 sum rounded once: against the fp64 sum, the
    error is at most the bf16 half-ulp plus the fp32 summation bound (n - 1) * 2^-24 * sum|y|; and
    against the fp32 sums it reports, the relative error is the bf16 rounding alone (< 2^-8)."""
    S, T, H, E, R, K, C = 4, 64, 512, 64, 16, 8, 4
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 17)
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C)
    y = wl.bf16_bits(wl.expert_outputs(r["num_recv"], H, seed=3))
    c = oracle.relay_combine(y, None, r["recv_rank_offset"], r["recv_rdma_offset"], r["send_nvl_head"],
                             r["send_rdma_head"], S=S, partial_f32=True, want_f32=True, want_f64=True)
    got = oracle.bf16_to_f32(c["combined_x"]).reshape(S * T, H).astype(np.float64)
    f32 = c["combined_f32"].astype(np.float64)
    f64 = c["combined_f64"]
    assert (np.abs(got - f32) / np.maximum(np.abs(f32), 1e-30)).max() <= 2.0 ** -8
    # sum of |y| per token, built from the dispatch's own rows
    absy = np.zeros((S * T, H))
    yf = np.abs(oracle.bf16_to_f32(y).reshape(y.shape).astype(np.float64))
    d = oracle.dispatch(np.zeros((S * T, 8), np.uint16), idx, None, itr, None, S=S, E=E, R=R, C=C)
    for n in range(S * T):
        for rr in range(R):
            j = d["send_head"][n, rr]
            if j >= 0:
                absy[n] += yf[d["recv_rank_offset"][rr] + j]
    cnt = itr.sum(axis=1)[:, None]
    bound = 2.0 ** -8 * np.abs(f64) + np.maximum(cnt - 1, 0) * 2.0 ** -24 * absy * 1.001
    assert np.all(np.abs(got - f64) <= bound)


def test_relay_combine_identity_and_weights():
    S, T, H, E, R, K, C = 4, 64, 512, 64, 16, 8, 4
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 11)
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C)
    c = oracle.relay_combine(r["recv_x"], r["recv_topk_weights"], r["recv_rank_offset"], r["recv_rdma_offset"],
                             r["send_nvl_head"], r["send_rdma_head"], S=S, want_f64=True)
    cnt = itr.sum(axis=1).astype(np.float64)
    got = (c["combined_x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = cnt > 0
    assert oracle.calc_diff(got[ok] / cnt[ok, None], xf[ok]) < 5e-6
    # the weight of entry k lives on one rank only: both levels add zeros to it
    valid = (idx >= 0) & ok[:, None]
    assert np.array_equal(c["combined_topk_weights"][valid], wts[valid])
    # fp64 reference is the exact multiple of x
    assert np.allclose(c["combined_f64"][ok], xf[ok] * cnt[ok, None], rtol=0, atol=0)


def test_relay_combine_equals_flat_when_one_rank_per_group():
    """A token reaching at most one rank of each group has single-term partials (exact in bf16), so the
    two-level sum is the flat combine bit for bit."""
    S, T, H, R, K = 2, 50, 256, 32, 4
    E = R                                             # one expert per rank
    g = torch.Generator().manual_seed(4)
    idx = np.empty((S * T, K), np.int64)
    for n in range(S * T):
        groups = torch.randperm(R // 8, generator=g)[:K].numpy()
        lanes = torch.randint(0, 8, (K,), generator=g).numpy()
        idx[n] = groups * 8 + lanes
    x = wl.bf16_bits(wl.activations(S * T, H, g))
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    assert itr.reshape(S * T, R // 8, 8).sum(axis=2).max() == 1
    r = oracle.relay_dispatch(x, idx, None, itr, S=S, E=E, R=R, C=3)
    y = wl.bf16_bits(wl.expert_outputs(r["num_recv"], H, seed=2))
    c = oracle.relay_combine(y, None, r["recv_rank_offset"], r["recv_rdma_offset"], r["send_nvl_head"],
                             r["send_rdma_head"], S=S)
    lay = oracle.layout(idx, S, E, R)
    d = oracle.dispatch(x, idx, None, itr, lay["num_tokens_per_expert"], S=S, E=E, R=R, C=3)
    f = oracle.combine(y, None, d["send_head"], d["recv_rank_offset"], S=S)
    assert np.array_equal(c["combined_x"], f["combined_x"])
    c32 = oracle.relay_combine(y, None, r["recv_rank_offset"], r["recv_rdma_offset"], r["send_nvl_head"],
                               r["send_rdma_head"], S=S, partial_f32=True)
    assert np.array_equal(c32["combined_x"], f["combined_x"])


def test_relay_combine_bias_added_last():
    S, T, H, E, R, K, C = 2, 20, 128, 32, 16, 4, 2
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 13)
    idx[::5] = -1                                     # tokens without any group
    itr = oracle.layout(idx, S, E, R)["is_token_in_rank"]
    r = oracle.relay_dispatch(x, idx, wts, itr, S=S, E=E, R=R, C=C)
    y = np.zeros((r["num_recv"], H), np.uint16)
    b = wl.bf16_bits(wl.activations(S * T, H, torch.Generator().manual_seed(1)))
    c = oracle.relay_combine(y, None, r["recv_rank_offset"], r["recv_rdma_offset"], r["send_nvl_head"],
                             r["send_rdma_head"], S=S, bias0=b)
    assert np.array_equal(c["combined_x"], b)         # 0 + b = b exactly, also for tokens no rank received
