"""Randomised GPU parity sweep: seeded random shapes and routings (one fixed
list, so every run sees the same cases) through the C ABI against the CPU
oracle, bit for bit: layout + dispatch + combine (bf16, FP8 cast, pre-quantised
FP8, worst-case capacity, bias), the low-latency dispatch + combine (masked
ranks, slot cap) and the relay."""
import sys

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_histogram_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_get_dispatch_histogram_amd as miep  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def npy(t):
    return t.detach().cpu().numpy()


def _routing(rng, N, E, K, mask_p, dup_p, oob_p):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int64) if N else np.zeros((0, K), np.int64)
    if N and K > 1 and dup_p:
        d = rng.random(N) < dup_p
        idx[d, 1] = idx[d, 0]
    if N and mask_p:
        idx[rng.random((N, K)) < mask_p] = -1
    if N and oob_p:
        idx[rng.random((N, K)) < oob_p] = E + 7
    return idx


def _normal_cases(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 32, 64, 128]))
        L = int(rng.integers(1, 5))
        E = R * L
        K = int(rng.integers(1, min(E, 9) + 1))
        S = int(rng.integers(1, 6))
        T = int(rng.integers(0, 300))
        C = int(rng.integers(1, 30))
        kind = ["bf16", "cast", "fp8"][i % 3]
        H = int(rng.choice([128, 256, 384, 1024])) if kind != "bf16" else int(8 * rng.integers(1, 200))
        out.append(dict(i=i, R=R, E=E, K=K, S=S, T=T, C=C, H=H, kind=kind, seed=int(rng.integers(0, 2 ** 31)),
                        mask_p=float(rng.choice([0.0, 0.15])), dup_p=float(rng.choice([0.0, 0.2])),
                        oob_p=float(rng.choice([0.0, 0.05])), worst=bool(rng.random() < 0.3),
                        bias=bool(rng.random() < 0.4), round_scale=bool(rng.random() < 0.5)))
    return out


def _channel_group_cases(n=40, seed=77):
    """Shapes of the channel-group notify (8/16/32/64 ranks, T * R a multiple of 16, channels of up to 256
    tokens): channel groups that start on odd tokens, many sources, one-token channels, multi-wavefront
    channels."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([8, 16, 32, 64]))
        L = int(rng.integers(1, 4))
        E = R * L
        K = int(rng.integers(1, min(E, 9) + 1))
        S = int(rng.choice([1, 3, 17, 70]))
        T = int(rng.integers(1, 400))
        if R == 8:
            T += T % 2                            # T * R % 16 == 0
        C = int(rng.choice([1, 2, 5, 7, 24, 41, T]))
        kind = ["bf16", "cast", "fp8"][i % 3]
        H = int(rng.choice([128, 256])) if kind != "bf16" else int(8 * rng.integers(1, 40))
        out.append(dict(i=100 + i, R=R, E=E, K=K, S=S, T=T, C=C, H=H, kind=kind, seed=int(rng.integers(0, 2 ** 31)),
                        mask_p=float(rng.choice([0.0, 0.15])), dup_p=float(rng.choice([0.0, 0.2])),
                        oob_p=float(rng.choice([0.0, 0.05])), worst=bool(rng.random() < 0.3),
                        bias=False, round_scale=bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", _normal_cases() + _channel_group_cases(),
                         ids=lambda c: "n%d-%s-R%d" % (c["i"], c["kind"], c["R"]))
def test_fuzz_normal(case):
    say("fuzz normal", case)
    c = case
    rng = np.random.default_rng(c["seed"])
    S, T, R, E, K, C, H = c["S"], c["T"], c["R"], c["E"], c["K"], c["C"], c["H"]
    N = S * T
    idx = _routing(rng, N, E, K, c["mask_p"], c["dup_p"], c["oob_p"])
    g = torch.Generator().manual_seed(c["seed"])
    x = wl.activations(N, H, g)
    wts = wl.gate_weights(N, K, g) if N else torch.zeros((0, K))
    idxd = torch.from_numpy(idx).to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    lay = oracle.layout(idx, S, E, R)
    xb = wl.bf16_bits(x)
    total = int(lay["num_tokens_per_rank"].sum())
    worst = total + 17 if c["worst"] else 0
    kw = {}
    okw = {}
    if c["kind"] == "cast":
        kw = dict(cast_to_fp8=True, round_scale=c["round_scale"])
        okw = dict(x_kind=oracle.X_BF16_CAST_FP8, round_scale=c["round_scale"])
        xin = x.to(DEV)
    elif c["kind"] == "fp8":
        codes, sci, _ = oracle.fp8_quantize(xb, round_scale=False)
        xin = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(DEV)
        kw = dict(x_scales=torch.from_numpy(sci).to(DEV))
        okw = dict(x_kind=oracle.X_FP8, x_scales=sci)
        xb = codes
    else:
        xin = x.to(DEV)
    recv_x, recv_s, rti, rtw, nrte, h = miep.dispatch(xin, idxd, wts.to(DEV), ntpr, itr, ntpe, E, C,
                                                      num_worst_tokens=worst, **kw)
    ref = oracle.dispatch(xb, idx, wts.numpy(), lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=S, E=E,
                          R=R, C=C, capacity=worst if worst else None, **okw)
    torch.cuda.synchronize()
    assert np.array_equal(npy(ntpr), lay["num_tokens_per_rank"])
    assert np.array_equal(npy(h.send_head), ref["send_head"])
    assert np.array_equal(npy(h.rank_prefix_matrix), ref["rank_prefix_matrix"])
    assert np.array_equal(npy(h.channel_prefix_matrix), ref["channel_prefix_matrix"])
    assert np.array_equal(npy(h.recv_channel_prefix_matrix), ref["recv_channel_prefix_matrix"])
    assert np.array_equal(npy(h.recv_rank_offset), ref["recv_rank_offset"])
    n = ref["num_recv"]
    got_x = u16(recv_x) if c["kind"] == "bf16" else u8(recv_x)
    assert np.array_equal(got_x[:n], ref["recv_x"][:n])
    if c["kind"] != "bf16":
        assert np.array_equal(npy(recv_s)[:n].view(np.uint32), ref["recv_x_scales"][:n].view(np.uint32))
    assert np.array_equal(npy(rti)[:n], ref["recv_topk_idx"][:n])
    assert np.array_equal(npy(nrte), ref["num_recv_tokens_per_expert"])
    # combine of random expert outputs (rows past the total are never read)
    y = wl.activations(h.recv_capacity, H, g)
    b = wl.activations(N, H, g) if c["bias"] else None
    cx, cw = miep.combine(y.to(DEV), h, rtw, bias=None if b is None else b.to(DEV))
    assert np.array_equal(npy(rtw)[:n].view(np.uint32), ref["recv_topk_weights"][:n].view(np.uint32))
    assert ref["recv_topk_weights"].shape[0] == h.recv_capacity
    rc = oracle.combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=S,
                        bias0=None if b is None else wl.bf16_bits(b))
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))


def _ll_cases(n=30, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 4, 8, 16]))
        L = int(rng.integers(1, 5))
        E = R * L
        K = int(rng.integers(1, min(E, 9) + 1))
        M = int(rng.integers(1, 160))
        T = int(rng.integers(0, M + 1))
        fp8 = bool(rng.random() < 0.5)
        H = int(rng.choice([512, 1024])) if fp8 else int(8 * rng.integers(1, 150))
        out.append(dict(i=i, R=R, E=E, K=K, M=M, T=T, H=H, fp8=fp8, d=int(rng.integers(0, R)),
                        seed=int(rng.integers(0, 2 ** 31)), mask=bool(rng.random() < 0.4) and R > 1,
                        weighted=bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", _ll_cases(), ids=lambda c: "ll%d-R%d-M%d" % (c["i"], c["R"], c["M"]))
def test_fuzz_low_latency(case):
    say("fuzz ll", case)
    c = case
    rng = np.random.default_rng(c["seed"])
    R, E, K, M, T, H, d = c["R"], c["E"], c["K"], c["M"], c["T"], c["H"], c["d"]
    N = R * T
    idx = _routing(rng, N, E, K, 0.1, 0.2, 0.0)
    g = torch.Generator().manual_seed(c["seed"])
    x = wl.activations(N, H, g)
    mask = mref = None
    if c["mask"]:
        mref = np.zeros(R, np.int32)
        mref[rng.choice(R, size=max(1, R // 3), replace=False)] = 1
        mask = torch.from_numpy(mref).to(DEV)
    out = miep.low_latency_dispatch(x.to(DEV), torch.from_numpy(idx).to(DEV), M, E, d, R, c["fp8"], mask_buffer=mask)
    ref = oracle.ll_dispatch(wl.bf16_bits(x), idx, S=R, M=M, E=E, R=R, dest_rank=d, use_fp8=c["fp8"],
                             round_scale=False, use_ue8m0=False, mask=mref)
    torch.cuda.synchronize()
    assert np.array_equal(npy(out["packed_recv_layout_range"]), ref["packed_recv_layout_range"])
    assert np.array_equal(npy(out["packed_recv_count"]), ref["packed_recv_count"])
    L = E // R
    for l in range(L):
        n = ref["packed_recv_count"][l]
        assert np.array_equal(npy(out["packed_recv_src_info"])[l, :n], ref["packed_recv_src_info"][l, :n])
        got = u8(out["packed_recv_x"][l, :n]) if c["fp8"] else u16(out["packed_recv_x"][l, :n])
        assert np.array_equal(got, ref["packed_recv_x"][l, :n])
    y = wl.activations(L * R * M, H, g).view(L, R * M, H)
    w = wl.gate_weights(N, K, g) if c["weighted"] and N else None
    cx = miep.low_latency_combine(y.to(DEV), torch.from_numpy(idx).to(DEV), None if w is None else w.to(DEV),
                                  out["packed_recv_src_info"], out["packed_recv_layout_range"], M, E, d, R)
    rc = oracle.ll_combine(wl.bf16_bits(y), ref["packed_recv_src_info"], ref["packed_recv_layout_range"], idx, S=R,
                           M=M, E=E, R=R, dest_rank=d, topk_weights=None if w is None else w.numpy())
    assert np.array_equal(u16(cx), rc["combined_x"])


def _relay_cases(n=16, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([16, 24, 32, 64, 128]))
        L = int(rng.integers(1, 4))
        E = R * L
        K = int(rng.integers(1, min(E, 9) + 1))
        S = int(rng.integers(1, 5))
        T = int(rng.integers(1, 200))
        C = int(rng.integers(1, 25))
        cast = bool(rng.random() < 0.5)
        H = int(rng.choice([128, 512])) if cast else int(8 * rng.integers(1, 100))
        out.append(dict(i=i, R=R, E=E, K=K, S=S, T=T, C=C, H=H, cast=cast, seed=int(rng.integers(0, 2 ** 31))))
    return out


@pytest.mark.parametrize("case", _relay_cases(), ids=lambda c: "relay%d-R%d" % (c["i"], c["R"]))
def test_fuzz_relay(case):
    say("fuzz relay", case)
    c = case
    rng = np.random.default_rng(c["seed"])
    S, T, R, E, K, C, H = c["S"], c["T"], c["R"], c["E"], c["K"], c["C"], c["H"]
    N = S * T
    idx = _routing(rng, N, E, K, 0.15, 0.2, 0.05)
    g = torch.Generator().manual_seed(c["seed"])
    x = wl.activations(N, H, g)
    wts = wl.gate_weights(N, K, g)
    idxd = torch.from_numpy(idx).to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    recv_x, recv_s, rti, rtw, _, h, rh, rdma_x, _ = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma,
                                                                       itr, ntpe, E, C, cast_to_fp8=c["cast"])
    lay = oracle.layout(idx, S, E, R)
    ref = oracle.relay_dispatch(wl.bf16_bits(x), idx, wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R, C=C,
                                x_kind=oracle.X_BF16_CAST_FP8 if c["cast"] else oracle.X_BF16)
    torch.cuda.synchronize()
    assert np.array_equal(npy(rh.send_rdma_head), ref["send_rdma_head"])
    ng = ref["num_rdma_recv"]
    assert np.array_equal(npy(rh.send_nvl_head)[:ng], ref["send_nvl_head"][:ng])
    got = u8(recv_x) if c["cast"] else u16(recv_x)
    assert np.array_equal(got, ref["recv_x"])
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    y = wl.activations(h.recv_capacity, H, g)
    cx, cw = miep.relay_combine(y.to(DEV), h, rh, rtw)
    rc = oracle.relay_combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["recv_rank_offset"],
                              ref["recv_rdma_offset"], ref["send_nvl_head"], ref["send_rdma_head"], S=S)
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))
