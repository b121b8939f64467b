"""Property-based pins of the oracle: layout, dispatch, combine and the
low-latency combine against the independent brute force on random shapes and
routings drawn by hypothesis (masked, duplicated and out-of-range entries, R
not a power of two, empty channels, T = 0)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import brute

SETTINGS = dict(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])


@st.composite
def routings(draw):
    S = draw(st.integers(1, 4))
    T = draw(st.integers(0, 12))
    R = draw(st.sampled_from([1, 2, 3, 4, 6, 8, 16, 24]))
    L = draw(st.integers(1, 4))
    E = R * L
    K = draw(st.integers(1, min(E, 6)))
    C = draw(st.integers(1, 9))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    mask_p = draw(st.sampled_from([0.0, 0.2, 1.0]))
    dup_p = draw(st.sampled_from([0.0, 0.3]))
    oob_p = draw(st.sampled_from([0.0, 0.1]))
    rng = np.random.default_rng(seed)
    N = S * T
    idx = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int64) if N else np.zeros((0, K), np.int64)
    if N and K > 1 and dup_p:
        d = rng.random(N) < dup_p
        idx[d, 1] = idx[d, 0]
    if N and mask_p:
        idx[rng.random((N, K)) < mask_p] = -1
    if N and oob_p:
        idx[rng.random((N, K)) < oob_p] = E + int(rng.integers(0, 5))
    return S, T, E, R, K, C, idx, rng


@settings(**SETTINGS)
@given(routings())
def test_fuzz_layout_dispatch_combine(orc, case):
    S, T, E, R, K, C, idx, rng = case
    N, H = S * T, 8
    lay = orc.layout(idx, S, E, R)
    want = brute.layout(idx, S, E, R)
    assert lay["num_tokens_per_rank"].tolist() == want["num_tokens_per_rank"]
    assert lay["num_tokens_per_expert"].tolist() == want["num_tokens_per_expert"]
    assert lay["is_token_in_rank"].astype(int).tolist() == [list(map(int, r)) for r in want["is_token_in_rank"]]
    if R > 8:
        assert lay["num_tokens_per_rdma_rank"].tolist() == want["num_tokens_per_rdma_rank"]

    x = rng.integers(0, 65535, (N, H), dtype=np.uint16)
    w = rng.random((N, K)).astype(np.float32)
    d = orc.dispatch(x, idx, w, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=S, E=E, R=R, C=C)
    received, cpm, rpm, rcpm = brute.dispatch_plan(lay["is_token_in_rank"], S, C)
    assert np.array_equal(d["channel_prefix_matrix"], cpm)
    assert np.array_equal(d["rank_prefix_matrix"], rpm)
    assert np.array_equal(d["recv_channel_prefix_matrix"], rcpm)
    L = E // R
    row = 0
    for r in range(R):
        assert d["recv_rank_offset"][r] == row
        for j, (s, t) in enumerate(received[r]):
            n = s * T + t
            assert d["send_head"][n, r] == j and d["recv_src_idx"][row + j] == t
            assert np.array_equal(d["recv_x"][row + j], x[n])
            for k in range(K):
                e = int(idx[n, k])
                mine = 0 <= e < E and e // L == r
                assert d["recv_topk_idx"][row + j, k] == (e - r * L if mine else -1)
        row += len(received[r])

    y = brute.bf16_round_lib(rng.standard_normal((max(d["num_recv"], 0), H)).astype(np.float32)).reshape(-1, H)
    c = orc.combine(y, d["recv_topk_weights"], d["send_head"], d["recv_rank_offset"], S=S)
    for n in range(N):
        rows = [d["recv_rank_offset"][r] + d["send_head"][n, r] for r in range(R) if d["send_head"][n, r] >= 0]
        for h in range(H):
            acc = brute.combine_token([brute.bf16_value(int(y[g, h])) for g in rows])
            want_h = 0 if acc is None else int(brute.bf16_round_lib(np.array([acc], np.float32))[0])
            assert c["combined_x"][n, h] == want_h


@settings(**SETTINGS)
@given(routings(), st.integers(1, 12), st.booleans())
def test_fuzz_ll_combine(orc, case, M, weighted):
    S, T, E, R, K, C, idx, rng = case
    if T > M or S != R:
        S = R                                        # the low-latency path has one source per rank
        T = min(T, M)
        N = S * T
        idx = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int64) if N else np.zeros((0, K),
                                                                                                         np.int64)
    N, H = S * T, 8
    d = int(rng.integers(0, R))
    x = rng.integers(0, 65535, (N, H), dtype=np.uint16)
    ll = orc.ll_dispatch(x, idx, S=S, M=M, E=E, R=R, dest_rank=d, use_fp8=False, round_scale=False,
                         use_ue8m0=False)
    L = E // R
    y = brute.bf16_round_lib(rng.standard_normal((L * S * M, H)).astype(np.float32)).reshape(L, S * M, H)
    w = rng.random((N, K)).astype(np.float32) if weighted else None
    got = orc.ll_combine(y, ll["packed_recv_src_info"], ll["packed_recv_layout_range"], idx, S=S, M=M, E=E, R=R,
                         dest_rank=d, topk_weights=w)
    want, have = brute.ll_combine(y, ll["packed_recv_src_info"], ll["packed_recv_layout_range"], idx, S, M, E, R, d,
                                  weights=w)
    want_bits = np.where(have[:, None], brute.bf16_round_lib(want).reshape(N, H), 0).astype(np.uint16)
    assert np.array_equal(got["combined_x"], want_bits)
