"""GPU parity of the widened rows: combine bias, low-latency rank masking and
the mask helpers, and the low-latency combine -- the HIP path through the C
ABI against the CPU oracle.

Bar: bit-exact (same fp32 summation order, one bf16 rounding) for every
output, plus, for the low-latency combine at full size, calc_diff < 5e-6
against the oracle's fp64 sum.
"""
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


def npy(t):
    return t.detach().cpu().numpy()


# --------------------------------------------------------------------------- combine bias
BIAS_CASES = [
    # name, S, T, H, E, R, K, C
    ("tiny", 4, 32, 256, 16, 4, 4, 24),
    ("ragged", 3, 1500, 2056, 48, 6, 5, 7),
    ("r16", 4, 96, 512, 64, 16, 6, 24),
]


def _dispatch(w, x, idx, wts):
    """The GPU dispatch and, for the expected values, the oracle's own one of
    the same routing (its handle and received weights)."""
    idxd = idx.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    recv_x, _, rti, rtw, _, h = miep.dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, itr, ntpe, w.E, w.C)
    lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    ref = oracle.dispatch(np.zeros((w.N, 8), np.uint16), idx.numpy(), wts.numpy(), lay["is_token_in_rank"], None,
                          S=w.S, E=w.E, R=w.R, C=w.C)
    torch.cuda.synchronize()
    assert np.array_equal(npy(h.send_head), ref["send_head"])
    assert np.array_equal(npy(h.recv_rank_offset), ref["recv_rank_offset"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    return recv_x, rtw, h, ref


@pytest.mark.parametrize("case", BIAS_CASES, ids=[c[0] for c in BIAS_CASES])
@pytest.mark.parametrize("which", ["b0", "b1", "both"])
def test_combine_bias_small(case, which):
    name, S, T, H, E, R, K, C = case
    w = wl.NormalWorkload(name, S=S, T=T, H=H, E=E, R=R, K=K, C=C)
    say("combine bias", case, which)
    inp = wl.normal_inputs(w, 4)
    idx = inp["topk_idx"].clone()
    idx[::9] = -1                                     # tokens no rank receives: bias only
    _, rtw, h, ref = _dispatch(w, inp["x"], idx, inp["topk_weights"])
    g = torch.Generator().manual_seed(21)
    y = wl.activations(h.recv_capacity, H, g)
    b0 = wl.activations(w.N, H, g) if which in ("b0", "both") else None
    b1 = wl.activations(w.N, H, g) if which in ("b1", "both") else None
    cx, cw = miep.combine(y.to(DEV), h, rtw, bias=(None if b0 is None else b0.to(DEV),
                                                   None if b1 is None else b1.to(DEV)))
    rc = oracle.combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=S,
                        bias0=None if b0 is None else wl.bf16_bits(b0),
                        bias1=None if b1 is None else wl.bf16_bits(b1))
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))
    # a token no rank received combines to its bias (rounded once)
    only = wl.bf16_bits(b0 if b0 is not None else b1)[::9]
    if b0 is not None and b1 is not None:
        only = None
    if only is not None:
        assert np.array_equal(u16(cx)[::9], only)


def test_combine_bias_normal_single_tensor():
    w = wl.NORMAL
    say("combine bias normal", w.name)
    inp = wl.normal_inputs(w, 0)
    recv_x, rtw, h, ref = _dispatch(w, inp["x"], inp["topk_idx"], inp["topk_weights"])
    y = wl.expert_outputs(h.recv_capacity, w.H, seed=7)
    b = wl.activations(w.N, w.H, torch.Generator().manual_seed(8))
    cx, _ = miep.combine(y.to(DEV), h, None, bias=b.to(DEV))
    rc = oracle.combine(wl.bf16_bits(y), None, ref["send_head"], ref["recv_rank_offset"], S=w.S,
                        bias0=wl.bf16_bits(b))
    assert np.array_equal(u16(cx), rc["combined_x"])
    # unbiased call on the same buffers is unchanged by the bias path
    cx2, _ = miep.combine(y.to(DEV), h)
    rc2 = oracle.combine(wl.bf16_bits(y), None, ref["send_head"], ref["recv_rank_offset"], S=w.S)
    assert np.array_equal(u16(cx2), rc2["combined_x"])


def test_combine_bias_streamed():
    """Two bias rows of 137.6 MB each (9600 tokens x hidden 7168), past the
    128 MiB above which the combine loads a bias non-temporally: bit-exact
    as with the default policy."""
    w = wl.NormalWorkload("bias-stream", S=8, T=1200, H=7168, E=64, R=8, K=4, C=24)
    assert w.N * 2 * w.H > 128 << 20
    say("combine bias streamed", w.name)
    inp = wl.normal_inputs(w, 5)
    _, rtw, h, ref = _dispatch(w, inp["x"], inp["topk_idx"], inp["topk_weights"])
    g = torch.Generator().manual_seed(23)
    y = wl.activations(h.recv_capacity, w.H, g)
    b0 = wl.activations(w.N, w.H, g)
    b1 = wl.activations(w.N, w.H, g)
    cx, cw = miep.combine(y.to(DEV), h, rtw, bias=(b0.to(DEV), b1.to(DEV)))
    rc = oracle.combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=w.S,
                        bias0=wl.bf16_bits(b0), bias1=wl.bf16_bits(b1))
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))


# --------------------------------------------------------------------------- rank mask
def test_mask_helpers():
    say("mask helpers")
    m = torch.full((37,), 5, dtype=torch.int32, device=DEV)
    miep.clean_mask_buffer(m)
    assert int(m.abs().sum()) == 0
    miep.update_mask_buffer(m, 3, True)
    miep.update_mask_buffer(m, 36, True)
    miep.update_mask_buffer(m, 0, True)
    miep.update_mask_buffer(m, 0, False)
    q = miep.query_mask_buffer(m)
    ref = np.zeros(37, np.int32)
    ref[[3, 36]] = 1
    assert np.array_equal(npy(q), ref)
    assert q.data_ptr() != m.data_ptr()
    with pytest.raises(miep.MiepError):
        miep.update_mask_buffer(m, 37, True)


LL_MASK_CASES = [
    # name, R, T, M, H, E, K, d, masked ranks
    ("src-masked", 4, 6, 8, 512, 16, 3, 1, (2,)),
    ("dest-masked", 4, 6, 8, 512, 16, 3, 1, (1,)),
    ("ragged-two", 6, 300, 320, 1536, 24, 4, 5, (0, 3)),
    ("none-set", 6, 300, 320, 1536, 24, 4, 5, ()),
]


def _ll_routing(R, T, E, K, seed=11):
    g = torch.Generator().manual_seed(seed)
    idx = wl.topk_uniform(R * T, E, K, g)
    idx[::7, 0] = -1
    if K > 1:
        idx[::5, 1] = idx[::5, 0]          # duplicated expert: two messages, two rows
    return idx, g


@pytest.mark.parametrize("case", LL_MASK_CASES, ids=[c[0] for c in LL_MASK_CASES])
@pytest.mark.parametrize("use_fp8", [False, True], ids=["bf16", "fp8"])
def test_ll_dispatch_rank_mask(case, use_fp8):
    name, R, T, M, H, E, K, d, masked = case
    say("ll mask", case, use_fp8)
    idx, g = _ll_routing(R, T, E, K)
    x = wl.activations(R * T, H, g)
    mask = torch.zeros((R,), dtype=torch.int32, device=DEV)
    for r in masked:
        miep.update_mask_buffer(mask, r, True)
    out = miep.low_latency_dispatch(x.to(DEV), idx.to(DEV), M, E, d, R, use_fp8, mask_buffer=mask)
    mref = np.zeros(R, np.int32)
    mref[list(masked)] = 1
    ref = oracle.ll_dispatch(wl.bf16_bits(x), idx.numpy(), S=R, M=M, E=E, R=R, dest_rank=d, use_fp8=use_fp8,
                             round_scale=False, use_ue8m0=False, mask=mref)
    torch.cuda.synchronize()
    assert np.array_equal(npy(out["msg_count"]), ref["msg_count"])
    assert np.array_equal(npy(out["packed_recv_count"]), ref["packed_recv_count"])
    assert np.array_equal(npy(out["packed_recv_layout_range"]), ref["packed_recv_layout_range"])
    L = E // R
    for l in range(L):
        n = ref["packed_recv_count"][l]
        assert np.array_equal(npy(out["packed_recv_src_info"])[l, :n], ref["packed_recv_src_info"][l, :n])
        if use_fp8:
            assert np.array_equal(npy(out["packed_recv_x"][l, :n].view(torch.uint8)), ref["packed_recv_x"][l, :n])
        else:
            assert np.array_equal(u16(out["packed_recv_x"][l, :n]), ref["packed_recv_x"][l, :n])
    if d in masked:
        assert int(out["packed_recv_count"].sum()) == 0
    for s in masked:
        assert int(out["msg_count"][:, s].sum()) == 0


# --------------------------------------------------------------------------- low-latency combine
LL_COMBINE_CASES = [
    # name, R, T, M, H, E, K, d, masked ranks
    ("ll-tiny", 4, 6, 8, 512, 16, 3, 1, ()),
    ("ll-capped", 4, 40, 40, 256, 8, 4, 2, ()),       # 2 experts per rank: slots spill past M, dropped
    ("ll-ragged", 6, 300, 320, 1536, 24, 4, 5, ()),
    ("ll-masked", 6, 300, 320, 1536, 24, 4, 5, (0, 3)),
    ("ll-wide", 1, 200, 200, 7168, 12, 9, 0, ()),     # one rank, K = 9 local entries: two load batches
    ("ll-odd-row", 5, 64, 64, 1000, 10, 2, 4, ()),    # row of 125 vectors: a ragged slice
    ("ll-odd-wide", 4, 50, 64, 2120, 16, 4, 2, ()),   # row of 265 vectors: 4-vector slices, the last one partial
    ("ll-k1", 2, 100, 100, 256, 4, 1, 1, ()),         # 64 tokens per wavefront group
    ("ll-k64", 2, 16, 16, 256, 128, 64, 0, ()),       # one token per group
]


@pytest.mark.parametrize("case", LL_COMBINE_CASES, ids=[c[0] for c in LL_COMBINE_CASES])
@pytest.mark.parametrize("weighted", [False, True], ids=["sum", "weighted"])
def test_ll_combine_small(case, weighted):
    name, R, T, M, H, E, K, d, masked = case
    say("ll combine", case, weighted)
    idx, g = _ll_routing(R, T, E, K)
    if name == "ll-capped":
        # every entry on rank d: k -> local expert k % L, then entry 1 duplicates entry 0, so local
        # expert 0 gets 3 entries per token (120 > M slots: the tail is dropped) and expert 1 gets 40
        idx[:, :] = d * (E // R) + torch.arange(K, dtype=torch.int64)[None, :] % (E // R)
        idx[:, 1] = idx[:, 0]
    x = wl.activations(R * T, H, g)
    wts = wl.gate_weights(R * T, K, g)
    mask = None
    mref = None
    if masked:
        mask = torch.zeros((R,), dtype=torch.int32, device=DEV)
        for r in masked:
            miep.update_mask_buffer(mask, r, True)
        mref = np.zeros(R, np.int32)
        mref[list(masked)] = 1
    use_fp8 = H % 128 == 0 and name != "ll-wide"
    out = miep.low_latency_dispatch(x.to(DEV), idx.to(DEV), M, E, d, R, use_fp8, mask_buffer=mask)
    ref = oracle.ll_dispatch(wl.bf16_bits(x), idx.numpy(), S=R, M=M, E=E, R=R, dest_rank=d, use_fp8=use_fp8,
                             round_scale=False, use_ue8m0=False, mask=mref)
    torch.cuda.synchronize()
    assert np.array_equal(npy(out["packed_recv_layout_range"]), ref["packed_recv_layout_range"])
    L = E // R
    y = wl.activations(L * R * M, H, g).view(L, R * M, H)
    cx = miep.low_latency_combine(y.to(DEV), idx.to(DEV), wts.to(DEV) if weighted else None,
                                  out["packed_recv_src_info"], out["packed_recv_layout_range"], M, E, d, R)
    rc = oracle.ll_combine(wl.bf16_bits(y), ref["packed_recv_src_info"], ref["packed_recv_layout_range"],
                           idx.numpy(), S=R, M=M, E=E, R=R, dest_rank=d,
                           topk_weights=wts.numpy() if weighted else None)
    assert np.array_equal(u16(cx), rc["combined_x"])
    if name == "ll-capped":
        assert int(out["msg_count"].max()) == M          # the cap was reached
    if d in masked:
        assert int(cx.abs().sum()) == 0


@pytest.mark.parametrize("weighted", [False, True], ids=["sum", "weighted"])
def test_ll_combine_full_workload(weighted):
    w = wl.LL
    say("ll combine full", w.name, weighted)
    inp = wl.ll_inputs(w, 0)
    g = torch.Generator().manual_seed(12)
    wts = wl.gate_weights(w.N, w.K, g)
    idxd = inp["topk_idx"].to(DEV)
    out = miep.low_latency_dispatch(inp["x"].to(DEV), idxd, w.M, w.E, w.dest_rank, w.R, True)
    # the oracle's own receive layout of the same routing (the payload does not enter it)
    ref = oracle.ll_dispatch(np.zeros((w.N, 8), np.uint16), inp["topk_idx"].numpy(), S=w.S, M=w.M, E=w.E, R=w.R,
                             dest_rank=w.dest_rank, use_fp8=False)
    torch.cuda.synchronize()
    assert np.array_equal(npy(out["packed_recv_layout_range"]), ref["packed_recv_layout_range"])
    n = ref["packed_recv_count"]
    for l in range(w.L):
        assert np.array_equal(npy(out["packed_recv_src_info"])[l, :n[l]], ref["packed_recv_src_info"][l, :n[l]])
    y = wl.expert_outputs(w.L * w.R * w.M, w.H, seed=13).view(w.L, w.R * w.M, w.H)
    cx = miep.low_latency_combine(y.to(DEV), idxd, wts.to(DEV) if weighted else None, out["packed_recv_src_info"],
                                  out["packed_recv_layout_range"], w.M, w.E, w.dest_rank, w.R)
    rc = oracle.ll_combine(wl.bf16_bits(y), ref["packed_recv_src_info"], ref["packed_recv_layout_range"],
                           inp["topk_idx"].numpy(), S=w.S, M=w.M, E=w.E, R=w.R, dest_rank=w.dest_rank,
                           topk_weights=wts.numpy() if weighted else None, want_f64=True)
    got = u16(cx)
    assert np.array_equal(got, rc["combined_x"])
    f = cx.float().cpu().numpy().astype(np.float64)
    touched = np.abs(rc["combined_f64"]).sum(axis=1) > 0
    assert touched.any()
    assert oracle.calc_diff(f[touched], rc["combined_f64"][touched]) < 5e-6
    assert np.all(f[~touched] == 0)


def test_ll_identity_round_trip_full():
    """bf16 dispatch then combine of the packed rows themselves, unweighted:
    every token comes back times the number of its entries on rank d."""
    w = wl.LL
    say("ll identity round trip", w.name)
    inp = wl.ll_inputs(w, 1)
    idx = inp["topk_idx"]
    idxd = idx.to(DEV)
    out = miep.low_latency_dispatch(inp["x"].to(DEV), idxd, w.M, w.E, w.dest_rank, w.R, False)
    cx = miep.low_latency_combine(out["packed_recv_x"], idxd, None, out["packed_recv_src_info"],
                                  out["packed_recv_layout_range"], w.M, w.E, w.dest_rank, w.R)
    lo = w.dest_rank * w.L
    cnt = ((idx >= lo) & (idx < lo + w.L)).sum(dim=1).numpy().astype(np.float64)
    got = cx.float().cpu().numpy().astype(np.float64)
    xf = inp["x"].float().numpy().astype(np.float64)
    ok = cnt > 0
    assert ok.any()
    assert oracle.calc_diff(got[ok] / cnt[ok, None], xf[ok]) < 5e-6
    assert np.all(got[~ok] == 0)


def test_ll_combine_no_tokens():
    say("ll combine no tokens")
    R, M, H, E, K = 4, 8, 512, 16, 2
    L = E // R
    y = torch.zeros((L, R * M, H), dtype=torch.bfloat16, device=DEV)
    si = torch.zeros((L, R * M), dtype=torch.int32, device=DEV)
    lr = torch.zeros((L, R), dtype=torch.int64, device=DEV)
    idx = torch.empty((0, K), dtype=torch.int64, device=DEV)
    cx = miep.low_latency_combine(y, idx, None, si, lr, M, E, 0, R)
    torch.cuda.synchronize()
    assert tuple(cx.shape) == (0, H)
