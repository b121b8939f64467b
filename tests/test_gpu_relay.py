"""GPU parity of the two-level relay: relay dispatch (group rows, relay
handle, and the receive side) and the two-level combine, through the C ABI,
against the CPU oracle.  Bar: bit-exact for every output; the identity round
trip also within calc_diff < 5e-6."""
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


SHAPES = [
    # name, S, T, H, E, R, K, C
    ("r16", 4, 96, 512, 64, 16, 6, 24),
    ("r24-ragged", 3, 700, 1160, 48, 24, 5, 7),      # 3 groups (scalar send_rdma_head stores), ragged rows
    ("r64", 4, 128, 256, 256, 64, 8, 5),
    ("r256", 2, 64, 264, 2048, 256, 9, 3),           # 32 groups
]


def _inputs(S, T, H, E, R, K, C, seed, variant):
    w = wl.NormalWorkload("relay", S=S, T=T, H=H, E=E, R=R, K=K, C=C)
    inp = wl.normal_inputs(w, seed)
    idx = inp["topk_idx"].numpy().copy()
    if variant == "masked-dup-oob":
        rng = np.random.default_rng(seed)
        if K > 1:
            d = rng.random(w.N) < 0.2
            idx[d, 1] = idx[d, 0]
        idx[rng.random(idx.shape) < 0.2] = -1
        idx[rng.random(idx.shape) < 0.05] = E + 3
    return w, inp["x"], torch.from_numpy(idx), inp["topk_weights"]


def _check_relay_handle(rh, ref):
    assert np.array_equal(npy(rh.recv_rdma_offset), ref["recv_rdma_offset"])
    assert np.array_equal(npy(rh.send_rdma_head), ref["send_rdma_head"])
    assert np.array_equal(npy(rh.rdma_rank_prefix_matrix), ref["rdma_rank_prefix_matrix"])
    assert np.array_equal(npy(rh.rdma_channel_prefix_matrix), ref["rdma_channel_prefix_matrix"])
    assert np.array_equal(npy(rh.recv_rdma_channel_prefix_matrix), ref["recv_rdma_channel_prefix_matrix"])
    n = ref["num_rdma_recv"]
    assert np.array_equal(npy(rh.rdma_src_idx)[:n], ref["rdma_src_idx"][:n])
    assert np.array_equal(npy(rh.send_nvl_head)[:n], ref["send_nvl_head"][:n])


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
@pytest.mark.parametrize("variant", ["plain", "masked-dup-oob"])
def test_relay_dispatch_combine_small(case, variant):
    name, S, T, H, E, R, K, C = case
    say("relay", case, variant)
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 1, variant)
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    out = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C)
    recv_x, _, rti, rtw, nrte, h, rh, rdma_x, _ = out
    lay = oracle.layout(idx.numpy(), S, E, R)
    xb = wl.bf16_bits(x)
    ref = oracle.relay_dispatch(xb, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R, C=C)
    flat = oracle.dispatch(xb, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], lay["num_tokens_per_expert"],
                           S=S, E=E, R=R, C=C)
    torch.cuda.synchronize()
    _check_relay_handle(rh, ref)
    n = ref["num_rdma_recv"]
    assert np.array_equal(u16(rdma_x)[:n], ref["rdma_x"][:n])
    # the ranks' handle and receive side: the direct dispatch's
    assert np.array_equal(npy(h.send_head), flat["send_head"])
    assert np.array_equal(npy(h.rank_prefix_matrix), flat["rank_prefix_matrix"])
    assert np.array_equal(npy(h.recv_channel_prefix_matrix), flat["recv_channel_prefix_matrix"])
    assert np.array_equal(npy(h.recv_rank_offset), ref["recv_rank_offset"])
    assert np.array_equal(u16(recv_x), ref["recv_x"])
    assert np.array_equal(npy(h.recv_src_idx), ref["recv_src_idx"])
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(npy(nrte), flat["num_recv_tokens_per_expert"])
    # two-level combine of random expert outputs, with the weights and a bias
    g = torch.Generator().manual_seed(5)
    y = wl.activations(h.recv_capacity, H, g)
    b = wl.activations(w.N, H, g)
    cx, cw = miep.relay_combine(y.to(DEV), h, rh, rtw, bias=b.to(DEV))
    rc = oracle.relay_combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["recv_rank_offset"],
                              ref["recv_rdma_offset"], ref["send_nvl_head"], ref["send_rdma_head"], S=S,
                              bias0=wl.bf16_bits(b))
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))


@pytest.mark.parametrize("kind", ["cast", "cast-pow2", "fp8"])
def test_relay_fp8_kinds_small(kind):
    S, T, H, E, R, K, C = 3, 200, 1024, 64, 16, 6, 5
    say("relay fp8", kind)
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 2, "masked-dup-oob")
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    lay = oracle.layout(idx.numpy(), S, E, R)
    xb = wl.bf16_bits(x)
    round_scale = kind == "cast-pow2"
    if kind == "fp8":
        codes, sci, _ = oracle.fp8_quantize(xb, round_scale=False)
        xin = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(DEV)
        xs = torch.from_numpy(sci).to(DEV)
        out = miep.relay_dispatch(xin, idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C, x_scales=xs)
        ref = oracle.relay_dispatch(codes, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R,
                                    C=C, x_kind=oracle.X_FP8, x_scales=sci)
    else:
        out = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C, cast_to_fp8=True,
                                  round_scale=round_scale)
        ref = oracle.relay_dispatch(xb, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R, C=C,
                                    x_kind=oracle.X_BF16_CAST_FP8, round_scale=round_scale)
    recv_x, recv_s, rti, rtw, _, h, rh, rdma_x, rdma_s = out
    torch.cuda.synchronize()
    _check_relay_handle(rh, ref)
    n = ref["num_rdma_recv"]
    assert np.array_equal(u8(rdma_x)[:n], ref["rdma_x"][:n])
    assert np.array_equal(npy(rdma_s)[:n].view(np.uint32), ref["rdma_x_scales"][:n].view(np.uint32))
    assert np.array_equal(u8(recv_x), ref["recv_x"])
    assert np.array_equal(npy(recv_s).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])


def test_relay_large_workload_bf16_and_identity_round_trip():
    """The 64-rank workload (8 groups) through the relay with bf16 rows: every output against the oracle,
    then identity experts through the two-level combine: bit-exact, and calc_diff < 5e-6 after dividing by
    the number of receiving ranks."""
    w = wl.LARGE
    say("relay large bf16", w.name)
    inp = wl.normal_inputs(w, 0)
    x, idx, wts = inp["x"], inp["topk_idx"], inp["topk_weights"]
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    recv_x, _, rti, rtw, _, h, rh, rdma_x, _ = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma,
                                                                     itr, ntpe, w.E, w.C)
    lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    xb = wl.bf16_bits(x)
    ref = oracle.relay_dispatch(xb, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=w.S, E=w.E, R=w.R, C=w.C)
    torch.cuda.synchronize()
    _check_relay_handle(rh, ref)
    n = ref["num_rdma_recv"]
    assert np.array_equal(u16(rdma_x)[:n], ref["rdma_x"][:n])
    assert np.array_equal(u16(recv_x), ref["recv_x"])
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    cx, cw = miep.relay_combine(recv_x, h, rh, rtw)
    rc = oracle.relay_combine(ref["recv_x"], ref["recv_topk_weights"], ref["recv_rank_offset"],
                              ref["recv_rdma_offset"], ref["send_nvl_head"], ref["send_rdma_head"], S=w.S)
    assert np.array_equal(u16(cx), rc["combined_x"])
    cnt = lay["is_token_in_rank"].sum(axis=1).astype(np.float64)
    got = cx.float().cpu().numpy().astype(np.float64)
    ok = cnt > 0
    assert oracle.calc_diff(got[ok] / cnt[ok, None], x.float().numpy().astype(np.float64)[ok]) < 5e-6
    valid = (idx.numpy() >= 0) & ok[:, None]
    assert np.array_equal(npy(cw)[valid], wts.numpy()[valid])


def test_relay_large_workload_fp8_cast():
    """The 64-rank workload with the FP8 cast before the first hop, compared in full: the relay handle,
    every group row's codes and scales, every forwarded receive row, the ranks' handle and top-k metadata,
    against the oracle's relay dispatch of the pre-quantised rows (each source row quantised once, in
    threads; the CPU pins show the cast-once relay equals it); the receive side also equals the direct
    FP8-cast dispatch on the GPU."""
    w = wl.LARGE
    say("relay large fp8", w.name)
    inp = wl.normal_inputs(w, 0)
    x, idx, wts = inp["x"], inp["topk_idx"], inp["topk_weights"]
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    recv_x, recv_s, rti, rtw, _, h, rh, rdma_x, rdma_s = miep.relay_dispatch(
        xd, idxd, wd, ntpr, ntp_rdma, itr, ntpe, w.E, w.C, cast_to_fp8=True)
    direct = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, cast_to_fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(recv_x.view(torch.uint8), direct[0].view(torch.uint8))
    assert torch.equal(recv_s, direct[1])
    assert torch.equal(rti, direct[2])
    assert torch.equal(h.send_head, direct[5].send_head)
    del direct
    codes, sci, _ = oracle.fp8_quantize(wl.bf16_bits(x), round_scale=False, threads=16)
    lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    ref = oracle.relay_dispatch(codes, idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=w.S, E=w.E, R=w.R,
                                C=w.C, x_kind=oracle.X_FP8, x_scales=sci)
    _check_relay_handle(rh, ref)
    n = ref["num_rdma_recv"]
    assert rh.rdma_capacity == n and h.recv_capacity == ref["num_recv"]
    assert np.array_equal(u8(rdma_x), ref["rdma_x"])
    assert np.array_equal(npy(rdma_s).view(np.uint32), ref["rdma_x_scales"].view(np.uint32))
    assert np.array_equal(u8(recv_x), ref["recv_x"])
    assert np.array_equal(npy(recv_s).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(npy(h.recv_src_idx), ref["recv_src_idx"])
    assert np.array_equal(npy(h.recv_rank_offset), ref["recv_rank_offset"])


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_relay_combine_fp32_partials_small(shape):
    """fp32 partials between the two levels: group partials and the combined rows bit-exact against the
    oracle, weights exact."""
    name, S, T, H, E, R, K, C = shape
    say("relay combine fp32 partials", shape)
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 5, "masked-dup-oob")
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    out = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C)
    h, rh, rtw = out[5], out[6], out[3]
    lay = oracle.layout(idx.numpy(), S, E, R)
    ref = oracle.relay_dispatch(np.zeros((w.N, 8), np.uint16), idx.numpy(), wts.numpy(), lay["is_token_in_rank"],
                                S=S, E=E, R=R, C=C)
    torch.cuda.synchronize()
    _check_relay_handle(rh, ref)
    y = wl.expert_outputs(h.recv_capacity, H, seed=8)
    rdma_y = torch.empty((rh.rdma_capacity, H), dtype=torch.float32, device=DEV)
    rdma_w = torch.empty((rh.rdma_capacity, K), dtype=torch.float32, device=DEV)
    cx = torch.empty((w.N, H), dtype=torch.bfloat16, device=DEV)
    cw = torch.empty((w.N, K), dtype=torch.float32, device=DEV)
    miep.relay_combine_into(y.to(DEV), h, rh, rdma_y, cx, rtw, rdma_w, cw)
    rc = oracle.relay_combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["recv_rank_offset"],
                              ref["recv_rdma_offset"], ref["send_nvl_head"], ref["send_rdma_head"], S=S,
                              partial_f32=True)
    torch.cuda.synchronize()
    ng = ref["num_rdma_recv"]
    assert np.array_equal(npy(rdma_y)[:ng].view(np.uint32), rc["rdma_y"][:ng].view(np.uint32))
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))


@pytest.mark.parametrize("partial_f32", [False, True], ids=["bf16-partials", "fp32-partials"])
def test_relay_large_combine_random_outputs(partial_f32):
    """The 64-rank workload's two-level combine of random bf16 expert outputs, against the oracle's own
    handles: bit-exact; with fp32 partials also max relative error < 1e-2 against the oracle's fp32 sums
    and the fp32 summation bound against the fp64 sum (bf16 partials are rounded between the levels, so
    only their bit-exact parity is claimed)."""
    w = wl.LARGE
    say("relay large combine", partial_f32)
    inp = wl.normal_inputs(w, 0)
    x, idx, wts = inp["x"], inp["topk_idx"], inp["topk_weights"]
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    out = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, w.E, w.C)
    h, rh, rtw = out[5], out[6], out[3]
    del out
    lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    ref = oracle.relay_dispatch(np.zeros((w.N, 8), np.uint16), idx.numpy(), wts.numpy(), lay["is_token_in_rank"],
                                S=w.S, E=w.E, R=w.R, C=w.C)
    torch.cuda.synchronize()
    _check_relay_handle(rh, ref)
    y = wl.expert_outputs(h.recv_capacity, w.H, seed=4)
    cx, cw = miep.relay_combine(y.to(DEV), h, rh, rtw, partial_f32=partial_f32)
    ymax = float(y.abs().max())
    yb = wl.bf16_bits(y)
    del y
    rc = oracle.relay_combine(yb, ref["recv_topk_weights"], ref["recv_rank_offset"], ref["recv_rdma_offset"],
                              ref["send_nvl_head"], ref["send_rdma_head"], S=w.S, partial_f32=partial_f32,
                              want_f32=partial_f32, want_f64=partial_f32)
    got = u16(cx)
    assert np.array_equal(got, rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))
    if partial_f32:
        g = oracle.bf16_to_f32(got).reshape(got.shape).astype(np.float64)
        f32 = rc["combined_f32"].astype(np.float64)
        assert (np.abs(g - f32) / np.maximum(np.abs(f32), 1e-6)).max() < 1e-2
        # |g - f64| <= 2^-8 |f64| + (n - 1) 2^-24 sum|y|, with sum|y| <= n max|y| over the n contributions
        f64 = rc["combined_f64"]
        cnt = lay["is_token_in_rank"].sum(axis=1)[:, None].astype(np.float64)
        assert np.all(np.abs(g - f64) <= 2.0 ** -8 * np.abs(f64) + np.maximum(cnt - 1, 0) * cnt * ymax * 2.0 ** -24)


def test_relay_no_sources():
    say("relay empty")
    R, E, H, K = 16, 32, 256, 4
    idx = torch.empty((0, K), dtype=torch.int64, device=DEV)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idx, E, R, 2)
    recv_x, _, _, rtw, _, h, rh, _, _ = miep.relay_dispatch(x, idx, None, ntpr, ntp_rdma, itr, ntpe, E, 4)
    cx, _ = miep.relay_combine(torch.empty((0, H), dtype=torch.bfloat16, device=DEV), h, rh)
    torch.cuda.synchronize()
    assert int(h.recv_rank_offset[-1]) == 0 and int(rh.recv_rdma_offset[-1]) == 0
    assert cx.shape == (0, H)


@pytest.mark.parametrize("mode", ["worst-case", "overflow"])
def test_relay_capacities(mode):
    """Fixed capacities: larger than needed (rows past the totals hold in-range poison that must never be
    read or overwritten), or smaller (rows past a capacity are neither written nor forwarded) -- against the
    oracle run with the same capacities."""
    S, T, H, E, R, K, C = 3, 120, 256, 64, 16, 6, 5
    say("relay capacities", mode)
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 4, "plain")
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    total, gtotal = int(ntpr.sum()), int(ntp_rdma.sum())
    cap, rcap = (total + 37, gtotal + 53) if mode == "worst-case" else (total - 41, gtotal - 29)
    h = miep.Handle.allocate(itr, S, K, E, C, cap)
    rh = miep.RelayHandle.allocate(w.N, S, R, C, rcap, DEV)
    rh.send_nvl_head.fill_(0)            # in-range poison: a stray read would misplace rows, not fault
    rh.rdma_src_idx.fill_(0)
    recv_x = torch.full((cap, H), 3.0, dtype=torch.bfloat16, device=DEV)
    rdma_x = torch.full((rcap, H), 5.0, dtype=torch.bfloat16, device=DEV)
    rti = torch.full((cap, K), -9, dtype=torch.int64, device=DEV)
    rtw = torch.full((cap, K), 9.0, dtype=torch.float32, device=DEV)
    miep.relay_dispatch_into(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, ntpe, h, rh, rdma_x, recv_x,
                             recv_topk_idx=rti, recv_topk_weights=rtw)
    lay = oracle.layout(idx.numpy(), S, E, R)
    ref = oracle.relay_dispatch(wl.bf16_bits(x), idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R,
                                C=C, rdma_capacity=rcap, capacity=cap)
    torch.cuda.synchronize()
    assert int(rh.recv_rdma_offset[-1]) == gtotal and int(h.recv_rank_offset[-1]) == total
    ng, nr = min(gtotal, rcap), min(total, cap)
    assert np.array_equal(npy(rh.send_nvl_head)[:ng], ref["send_nvl_head"][:ng])
    assert np.array_equal(u16(rdma_x)[:ng], ref["rdma_x"][:ng])
    # the oracle leaves unwritten receive rows at zero: compare the rows it wrote
    written = np.zeros(cap, bool)
    off = ref["recv_rank_offset"]
    for r in range(R):
        for q in range(ref["recv_rank_offset"][r + 1] - off[r]):
            row = off[r] + q
            if row < cap:
                written[row] = (ref["recv_src_idx"][row] >= 0)
    assert np.array_equal(u16(recv_x)[written], ref["recv_x"][written])
    assert np.array_equal(npy(rti)[written], ref["recv_topk_idx"][written])
    # nothing else was touched
    assert np.all(u16(recv_x)[~written] == np.uint16(0x4040))       # bf16 3.0
    if mode == "worst-case":
        assert np.all(u16(rdma_x)[gtotal:] == np.uint16(0x40A0))    # bf16 5.0
        assert np.all(npy(rti)[total:] == -9)
    # the two-level combine on the same capacities
    y = wl.expert_outputs(cap, H, seed=6)
    cx, _ = miep.relay_combine(y.to(DEV), h, rh)
    rc = oracle.relay_combine(wl.bf16_bits(y), None, ref["recv_rank_offset"], ref["recv_rdma_offset"],
                              ref["send_nvl_head"], ref["send_rdma_head"], S=S)
    assert np.array_equal(u16(cx), rc["combined_x"])


@pytest.mark.parametrize("cast", [False, True], ids=["bf16", "fp8-cast"])
def test_relay_cached_dispatch(cast):
    """A new x through the handles of an earlier relay dispatch equals a fresh relay dispatch of it."""
    S, T, H, E, R, K, C = 4, 150, 512, 64, 32, 6, 5
    say("relay cached", cast)
    w, x, idx, wts = _inputs(S, T, H, E, R, K, C, 8, "masked-dup-oob")
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, E, R, S)
    out = miep.relay_dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C, cast_to_fp8=cast)
    h, rh = out[5], out[6]
    x2 = wl.activations(w.N, H, torch.Generator().manual_seed(77))
    recv2, recv2_s = miep.relay_cached_dispatch(x2.to(DEV), h, rh, cast_to_fp8=cast)
    fresh = miep.relay_dispatch(x2.to(DEV), idxd, wts.to(DEV), ntpr, ntp_rdma, itr, ntpe, E, C, cast_to_fp8=cast)
    lay = oracle.layout(idx.numpy(), S, E, R)
    ref = oracle.relay_dispatch(wl.bf16_bits(x2), idx.numpy(), wts.numpy(), lay["is_token_in_rank"], S=S, E=E, R=R,
                                C=C, x_kind=oracle.X_BF16_CAST_FP8 if cast else oracle.X_BF16)
    torch.cuda.synchronize()
    if cast:
        assert np.array_equal(u8(recv2), ref["recv_x"])
        assert np.array_equal(npy(recv2_s).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
        assert torch.equal(recv2.view(torch.uint8), fresh[0].view(torch.uint8))
    else:
        assert np.array_equal(u16(recv2), ref["recv_x"])
        assert torch.equal(recv2, fresh[0])
