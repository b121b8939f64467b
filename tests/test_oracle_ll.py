"""Pins for the oracle's low-latency dispatch (O7 send side, O8 receive side)."""
import numpy as np
import pytest
import torch

import brute
from combine_get_dispatch_histogram_amd import workloads as wl


def _case(S, T, M, H, E, K, seed, dup=False, mask_p=0.0):
    g = torch.Generator().manual_seed(seed)
    idx = wl.topk_uniform(S * T, E, K, g).numpy().copy()
    rng = np.random.default_rng(seed)
    if dup and K > 1:
        idx[::3, 1] = idx[::3, 0]
    if mask_p:
        idx[rng.random(idx.shape) < mask_p] = -1
    x = wl.bf16_bits(wl.activations(S * T, H, g))
    return x, idx


def _msg_used(H, use_fp8):
    # int4 header + (H FP8 bytes + H/128 fp32 scales) or 2H bf16 bytes
    return 16 + (H + (H // 128) * 4 if use_fp8 else 2 * H)


def _msg_bytes_formula(H, use_fp8):
    # the stride: rounded up to whole 16-byte pieces
    return -(-_msg_used(H, use_fp8) // 16) * 16


def test_msg_bytes(orc):
    assert orc.ll_msg_bytes(7168, True) == 7408 == 463 * 16
    assert orc.ll_msg_bytes(7168, False) == 14352
    assert orc.ll_msg_bytes(128, True) == 160          # 148 used bytes, 12 of padding
    assert orc.ll_msg_bytes(640, True) == 688          # 676 used
    for H in (128, 256, 384, 512, 640, 4096):
        for f in (True, False):
            assert orc.ll_msg_bytes(H, f) == _msg_bytes_formula(H, f)
            assert orc.ll_msg_bytes(H, f) % 16 == 0
            assert 0 <= orc.ll_msg_bytes(H, f) - _msg_used(H, f) < 16


@pytest.mark.parametrize("use_fp8,round_scale,use_ue8m0", [(False, False, False), (True, False, False),
                                                           (True, True, False), (True, True, True)])
@pytest.mark.parametrize("dup,mask_p", [(False, 0.0), (True, 0.2)])
@pytest.mark.parametrize("H", [256, 384])   # 384: FP8 messages with 4 bytes of padding
def test_ll_matches_brute(orc, use_fp8, round_scale, use_ue8m0, dup, mask_p, H):
    S = R = 4
    T, M, E, K, d = 6, 8, 16, 3, 1
    L = E // R
    x, idx = _case(S, T, M, H, E, K, 3, dup, mask_p)
    o = orc.ll_dispatch(x, idx, S=S, M=M, E=E, R=R, dest_rank=d, use_fp8=use_fp8, round_scale=round_scale,
                        use_ue8m0=use_ue8m0, cumulative_stats=np.full(L, 5, np.int32))
    mb = _msg_used(H, use_fp8)
    assert o["msg_buf"].shape[-1] == _msg_bytes_formula(H, use_fp8)
    for l in range(L):
        begin = 0
        for s in range(S):
            hits = [t for t in range(T) for k in range(K) if idx[s * T + t, k] == d * L + l]
            assert o["msg_count"][l, s] == len(hits)
            assert o["packed_recv_layout_range"][l, s] == (begin << 32) | len(hits)
            for j, t in enumerate(hits):
                msg = o["msg_buf"][l, s, j]
                assert msg[:16].view(np.int32).tolist() == [t, 0, 0, 0]
                row = begin + j
                assert o["packed_recv_src_info"][l, row] == t
                if use_fp8:
                    codes, scales, exps = brute.fp8_quantize_row(x[s * T + t], round_scale)
                    assert msg[16:16 + H].tolist() == codes
                    assert msg[16 + H:mb].view(np.float32).tolist() == [float(v) for v in scales]
                    assert o["packed_recv_x"][l, row].tolist() == codes
                    assert o["packed_recv_x_scales"][l, row].tolist() == [float(v) for v in scales]
                    if use_ue8m0:
                        assert o["packed_recv_x_scales_ue8m0"][l, row].tolist() == [e + 127 for e in exps]
                else:
                    assert np.array_equal(msg[16:mb].view(np.uint16), x[s * T + t])
                    assert np.array_equal(o["packed_recv_x"][l, row], x[s * T + t])
            begin += len(hits)
        assert o["packed_recv_count"][l] == begin
        assert o["cumulative_local_expert_recv_stats"][l] == 5 + begin


def test_ll_rejects_bad_flags(orc):
    x, idx = _case(2, 2, 2, 128, 4, 1, 0)
    with pytest.raises(ValueError):
        orc.ll_dispatch(x, idx, S=2, M=2, E=4, R=2, dest_rank=0, use_fp8=True, round_scale=False, use_ue8m0=True)
    with pytest.raises(ValueError):
        orc.ll_dispatch(x, idx, S=2, M=1, E=4, R=2, dest_rank=0, use_fp8=True)      # T > M


def test_ll_counts_full_size(orc):
    """Full LL workload: per-expert receive counts equal the layout's per-expert
    counts summed over sources; ~M*K/E = 4 messages per (expert, source)."""
    w = wl.LL
    inp = wl.ll_inputs(w, 0)
    idx = inp["topk_idx"].numpy()
    x = wl.bf16_bits(inp["x"])
    o = orc.ll_dispatch(x, idx, S=w.S, M=w.M, E=w.E, R=w.R, dest_rank=w.dest_rank, use_fp8=True, round_scale=True,
                        use_ue8m0=True)
    lay = orc.layout(idx, w.S, w.E, w.R)
    L = w.L
    want = lay["num_tokens_per_expert"][:, w.dest_rank * L:(w.dest_rank + 1) * L].sum(axis=0)
    assert np.array_equal(o["packed_recv_count"], want)
    assert abs(o["msg_count"].mean() - w.M * w.K / w.E) < 0.5
    # layout ranges tile [0, count) in source order
    lr = o["packed_recv_layout_range"]
    begin, n = lr >> 32, lr & 0xFFFFFFFF
    assert np.array_equal(begin[:, 0], np.zeros(L)) and np.array_equal(begin[:, 1:], (begin + n)[:, :-1])
    assert np.array_equal((begin + n)[:, -1], want)
    # every packed row dequantises close to the source row it names
    for l in range(L):
        for s in range(0, w.S, 7):
            for j in range(int(n[l, s])):
                row = int(begin[l, s]) + j
                t = o["packed_recv_src_info"][l, row]
                deq = orc.e4m3_decode(o["packed_recv_x"][l, row]) * np.repeat(o["packed_recv_x_scales"][l, row], 128)
                src = orc.bf16_to_f32(x[s * w.T + t])
                sc = np.repeat(o["packed_recv_x_scales"][l, row], 128)
                assert np.all(np.abs(deq - src) <= np.maximum(np.abs(src) * 2.0 ** -4, sc * 2.0 ** -10) * 1.0001)
