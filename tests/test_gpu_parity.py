"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for the layout, the handle (prefix matrices, offsets,
send_head, recv_src_idx), the received rows and top-k metadata, the FP8
codes and scales, and the low-latency messages and packed outputs.  Combine
is compared bit-exactly too (same summation order), and additionally held to
the stated tolerances: max relative error < 1e-2 against the fp32 reference
and, for identity experts, calc_diff < 5e-6 after dividing by the number of
receiving ranks.  Full-size workloads are compared in full, FP8 payloads
included.  Every expected value comes from the oracle run on its own
inputs (its own handle and weights), never from a GPU output.
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


def u8(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def npy(t):
    return t.detach().cpu().numpy()


def _inputs(w, seed=0):
    inp = wl.normal_inputs(w, seed)
    return inp["x"], inp["topk_idx"], inp["topk_weights"]


def _ref_dispatch(w, x_bits, idx, wts, lay, **kw):
    return oracle.dispatch(x_bits, idx, wts, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=w.S, E=w.E,
                           R=w.R, C=w.C, expert_alignment=w.expert_alignment, **kw)


def _check_layout(w, idx_t, got):
    ntpr, ntp_rdma, ntpe, itr = got
    ref = oracle.layout(npy(idx_t), w.S, w.E, w.R)
    assert np.array_equal(npy(ntpr), ref["num_tokens_per_rank"])
    assert np.array_equal(npy(ntpe), ref["num_tokens_per_expert"])
    assert np.array_equal(npy(itr).astype(np.uint8), ref["is_token_in_rank"])
    if w.R > 8:
        assert np.array_equal(npy(ntp_rdma), ref["num_tokens_per_rdma_rank"])
    else:
        assert ntp_rdma is None
    return ref


def _check_handle(h, ref):
    assert np.array_equal(npy(h.rank_prefix_matrix), ref["rank_prefix_matrix"])
    assert np.array_equal(npy(h.channel_prefix_matrix), ref["channel_prefix_matrix"])
    assert np.array_equal(npy(h.recv_channel_prefix_matrix), ref["recv_channel_prefix_matrix"])
    assert np.array_equal(npy(h.recv_rank_offset), ref["recv_rank_offset"])
    assert np.array_equal(npy(h.send_head), ref["send_head"])
    n = min(ref["num_recv"], h.recv_capacity)
    assert np.array_equal(npy(h.recv_src_idx)[:n], ref["recv_src_idx"][:n])


SMALL = [
    # name, S, T, H, E, R, K, C, align
    ("tiny", 4, 32, 256, 16, 4, 4, 24, 1),
    ("ragged", 3, 1500, 2056, 48, 6, 5, 7, 4),       # 2 token tiles, R % 4 != 0, ragged row tail
    ("one-src", 1, 700, 7168, 64, 8, 8, 24, 1),
    ("r16", 4, 96, 512, 64, 16, 6, 24, 2),            # two RDMA groups
    ("r128", 2, 100, 256, 1024, 128, 8, 5, 1),        # 2-word rank masks
    ("r256", 2, 64, 264, 2048, 256, 9, 3, 1),
    ("r1", 2, 40, 128, 8, 1, 2, 4, 1),
    ("k20", 2, 50, 128, 64, 8, 20, 4, 1),            # top-20: the pack writes the receive metadata
    ("r8-tiles", 2, 1300, 64, 32, 8, 4, 24, 2),      # 8-byte membership rows, 2 token tiles in the notify
    ("r40", 2, 300, 64, 80, 40, 6, 9, 1),            # bit-transpose notify: 10 of 16 lanes per token row
    ("r24-tiles", 2, 1100, 64, 96, 24, 6, 7, 1),     # bit-transpose notify over 2 token tiles
    ("r64-tiles", 1, 1100, 64, 128, 64, 4, 24, 1),   # 64 ranks, 2 token tiles, one source
    ("many-src", 40, 32, 64, 16, 4, 4, 5, 1),        # notify: > 16 sources per wavefront (batched count rows)
    ("many-src-r16", 33, 16, 64, 32, 16, 4, 3, 1),   # the same on the bit-transpose path
    ("huge-T", 1, (1 << 20) + 7, 8, 2, 2, 1, 3, 1),  # > 2^20 tokens per source: channel index by plain division
    ("rec-1024", 2, 1024, 64, 64, 16, 8, 24, 1),     # longest sources written by the record wavefronts
    ("rec-1025", 2, 1025, 64, 64, 16, 8, 24, 1),     # one token more: the records go back inline
    ("rec-k64", 3, 130, 64, 256, 8, 64, 5, 1),       # top-64: one record row per store instruction
    ("rec-k20-r64", 2, 200, 64, 128, 64, 20, 7, 1),  # 3 rows per store, 64 ranks, four 64-token chunks
    ("rec-parts", 3, 1000, 64, 64, 8, 16, 24, 1),    # 16 record wavefronts per (source, rank), ~29 parts: two each
    ("rec-parts-r16", 2, 700, 64, 128, 16, 12, 24, 1),  # 14 record wavefronts, parts of 40 rows, ragged last
    ("chan-odd", 3, 210, 64, 64, 8, 4, 10, 1),       # channel groups of 3 x 21 tokens: odd first token (half piece)
    ("chan-2wave", 2, 512, 64, 64, 32, 6, 4, 1),     # 128-token channels: two wavefronts per workgroup
    ("chan-many-src", 70, 32, 64, 512, 8, 6, 4, 1),  # > 64 sources, > 4 experts per workgroup
    ("chan-r32", 4, 160, 64, 128, 32, 8, 24, 2),     # 32 ranks: 9 channels of 7 tokens per workgroup
]


def _small_workload(name, S, T, H, E, R, K, C, align, **kw):
    return wl.NormalWorkload(name, S=S, T=T, H=H, E=E, R=R, K=K, C=C, expert_alignment=align, **kw)


def _masked_inputs(w, seed, mask_p=0.0, dup_p=0.0, oob_p=0.0):
    x, idx, wts = _inputs(w, seed)
    rng = np.random.default_rng(seed)
    idx = idx.numpy().copy()
    if dup_p and w.K > 1:
        d = rng.random(w.N) < dup_p
        idx[d, 1] = idx[d, 0]
    if mask_p:
        idx[rng.random(idx.shape) < mask_p] = -1
    if oob_p:
        idx[rng.random(idx.shape) < oob_p] = w.E + 3
    return x, torch.from_numpy(idx), wts


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("variant", ["plain", "masked-dup-oob"])
def test_layout_dispatch_combine_small(case, variant):
    w = _small_workload(*case)
    say("layout/dispatch/combine", case, variant)
    if variant == "plain":
        x, idx, wts = _inputs(w, 1)
    else:
        x, idx, wts = _masked_inputs(w, 2, mask_p=0.2, dup_p=0.2, oob_p=0.05)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    lay = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    ref_lay = _check_layout(w, idx, lay)
    ntpr, _, ntpe, itr = lay
    recv_x, _, rti, rtw, nrte, h = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, w.expert_alignment)
    ref = _ref_dispatch(w, wl.bf16_bits(x), idx.numpy(), wts.numpy(), ref_lay)
    torch.cuda.synchronize()
    _check_handle(h, ref)
    assert np.array_equal(u16(recv_x), ref["recv_x"])
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(npy(nrte), ref["num_recv_tokens_per_expert"])
    # combine of random expert outputs: bit-exact against the oracle (same order)
    y = wl.expert_outputs(h.recv_capacity, w.H, seed=5)
    cx, cw = miep.combine(y.to(DEV), h, rtw)
    rc = oracle.combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=w.S,
                        want_f32=True)
    assert np.array_equal(u16(cx), rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))


@pytest.mark.parametrize("wname", ["tiny", "normal", "skewed"])
def test_full_workload_bf16(wname):
    """Full-size normal / skewed workloads: every output bit-exact, identity
    round trip and random-y combine within the stated tolerances."""
    w = wl.WORKLOADS[wname]
    say("full bf16", wname)
    x, idx, wts = _inputs(w, 0)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    lay = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    ref_lay = _check_layout(w, idx, lay)
    if wname != "skewed":
        # per-expert counts sum to the valid top-k entries
        assert int(lay[2].sum()) == int((idx >= 0).sum())
    ntpr, _, ntpe, itr = lay
    recv_x, _, rti, rtw, nrte, h = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C)
    x_bits = wl.bf16_bits(x)
    ref = _ref_dispatch(w, x_bits, idx.numpy(), wts.numpy(), ref_lay)
    torch.cuda.synchronize()
    _check_handle(h, ref)
    assert np.array_equal(u16(recv_x), ref["recv_x"])
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(npy(nrte), ref["num_recv_tokens_per_expert"])

    # identity experts: combined / (#ranks that received the token) == x
    cx, cw = miep.combine(recv_x, h, rtw)
    rc = oracle.combine(ref["recv_x"], ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=w.S)
    assert np.array_equal(u16(cx), rc["combined_x"])
    cnt = ref_lay["is_token_in_rank"].sum(axis=1).astype(np.float64)
    got = cx.float().cpu().numpy().astype(np.float64)
    xf = x.float().numpy().astype(np.float64)
    ok = cnt > 0
    assert oracle.calc_diff(got[ok] / cnt[ok, None], xf[ok]) < 5e-6
    assert np.all(got[~ok] == 0)
    valid = (idx.numpy() >= 0) & ok[:, None]
    assert np.array_equal(npy(cw)[valid], wts.numpy()[valid])

    # random expert outputs: max relative error vs the fp32 reference < 1e-2
    y = wl.expert_outputs(h.recv_capacity, w.H, seed=3)
    cy, _ = miep.combine(y.to(DEV), h)
    ry = oracle.combine(wl.bf16_bits(y), None, ref["send_head"], ref["recv_rank_offset"], S=w.S, want_f32=True)
    assert np.array_equal(u16(cy), ry["combined_x"])
    g = cy.float().cpu().numpy().astype(np.float64)
    f = ry["combined_f32"].astype(np.float64)
    assert (np.abs(g - f) / np.maximum(np.abs(f), 1e-6)).max() < 1e-2


def test_cached_dispatch_normal():
    w = wl.NORMAL
    say("cached dispatch", w.name)
    x, idx, wts = _inputs(w, 0)
    idxd = idx.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    _, _, _, _, _, h = miep.dispatch(x.to(DEV), idxd, wts.to(DEV), ntpr, itr, ntpe, w.E, w.C)
    x2 = wl.activations(w.N, w.H, torch.Generator().manual_seed(9))
    recv2, _ = miep.cached_dispatch(x2.to(DEV), h)
    # the oracle's own handle, from its own layout and dispatch of the routing
    lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    d = oracle.dispatch(np.zeros((w.N, 8), np.uint16), idx.numpy(), None, lay["is_token_in_rank"], None, S=w.S,
                        E=w.E, R=w.R, C=w.C)
    ref = oracle.cached_dispatch(wl.bf16_bits(x2), d["send_head"], d["recv_rank_offset"], S=w.S,
                                 capacity=d["num_recv"])
    assert h.recv_capacity == d["num_recv"]
    assert np.array_equal(u16(recv2), ref["recv_x"])


def test_capacity_guard_and_worst_case_mode():
    """Worst-case capacity: the true total is reported, rows past the
    capacity are never written (guard rows stay intact), and the device
    status word reads MIEP_ECAPACITY exactly when the capacity is too small."""
    w = _small_workload("cap", 2, 300, 512, 32, 4, 4, 6, 1)
    say("capacity guard", w)
    x, idx, wts = _inputs(w, 4)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    total = int(ntpr.sum())
    ref = oracle.dispatch(wl.bf16_bits(x), idx.numpy(), wts.numpy(), npy(itr).astype(np.uint8), npy(ntpe), S=w.S,
                          E=w.E, R=w.R, C=w.C)
    for cap in (total // 2, total, w.N * w.R):
        guard = 64
        h = miep.Handle.allocate(itr, w.S, w.K, w.E, w.C, cap)
        recv_x = torch.full((cap + guard, w.H), 7.0, dtype=torch.bfloat16, device=DEV)
        rti = torch.full((cap + guard, w.K), 123, dtype=torch.int64, device=DEV)
        rtw = torch.full((cap + guard, w.K), 5.0, dtype=torch.float32, device=DEV)
        status = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        miep.dispatch_into(xd, idxd, wd, ntpr, ntpe, h, recv_x, None, rti, rtw, None, status=status)
        torch.cuda.synchronize()
        n = min(cap, total)
        assert int(h.recv_rank_offset[-1]) == total
        assert int(status) == (miep.MIEP_ECAPACITY if total > cap else 0)
        if total > cap:
            with pytest.raises(miep.MiepError) as err:
                miep.check_status(status)
            assert err.value.status == miep.MIEP_ECAPACITY
        else:
            miep.check_status(status)
        assert np.array_equal(u16(recv_x[:n]), ref["recv_x"][:n])
        assert np.array_equal(npy(rti[:n]), ref["recv_topk_idx"][:n])
        assert bool((recv_x[cap:] == 7.0).all()) and bool((rti[cap:] == 123).all()) and bool((rtw[cap:] == 5).all())
        if cap > total:
            assert bool((recv_x[total:] == 7.0).all())
        assert np.array_equal(npy(h.send_head), ref["send_head"])
    # the allocating call raises on an overflow (its synchronous check), and not otherwise
    with pytest.raises(miep.MiepError) as err:
        miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, num_worst_tokens=total - 1)
    assert err.value.status == miep.MIEP_ECAPACITY
    out = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, num_worst_tokens=total)
    assert int(out[5].recv_rank_offset[-1]) == total
    # no sources: the status is cleared
    st = torch.full((1,), 4, dtype=torch.int32, device=DEV)
    e = torch.empty((0, w.K), dtype=torch.int64, device=DEV)
    z = _small_workload("cap0", 2, 0, 512, 32, 4, 4, 6, 1)
    ntpr0, _, ntpe0, itr0 = miep.get_dispatch_layout(e, z.E, z.R, z.S)
    h0 = miep.Handle.allocate(itr0, z.S, z.K, z.E, z.C, 4)
    miep.dispatch_into(torch.empty((0, z.H), dtype=torch.bfloat16, device=DEV), e, None, ntpr0, ntpe0, h0,
                       torch.empty((4, z.H), dtype=torch.bfloat16, device=DEV), status=st)
    torch.cuda.synchronize()
    assert int(st) == 0


def test_empty_inputs():
    say("empty: T = 0")
    w = _small_workload("empty", 4, 0, 256, 16, 4, 4, 24, 1)
    idx = torch.empty((0, w.K), dtype=torch.int64, device=DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idx, w.E, w.R, w.S)
    assert int(ntpr.abs().sum()) == 0 and int(ntpe.abs().sum()) == 0
    x = torch.empty((0, w.H), dtype=torch.bfloat16, device=DEV)
    recv_x, _, rti, rtw, nrte, h = miep.dispatch(x, idx, torch.empty((0, w.K), device=DEV), ntpr, itr, ntpe, w.E,
                                                 w.C)
    torch.cuda.synchronize()
    assert recv_x.shape[0] == 0
    assert npy(h.recv_rank_offset).tolist() == [0] * (w.R + 1)
    assert int(h.channel_prefix_matrix.abs().sum()) == 0 and int(h.rank_prefix_matrix.abs().sum()) == 0
    assert int(nrte.abs().sum()) == 0
    cx, cw = miep.combine(torch.empty((0, w.H), dtype=torch.bfloat16, device=DEV), h, rtw)
    assert cx.shape == (0, w.H)


def test_all_masked_tokens_combine_to_zero():
    w = _small_workload("masked", 2, 64, 256, 16, 4, 4, 3, 1)
    say("all masked", w)
    x, idx, wts = _inputs(w, 6)
    idx = idx.clone()
    idx[::2] = -1                          # every other token goes nowhere
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    recv_x, _, rti, rtw, _, h = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C)
    cx, cw = miep.combine(recv_x, h, rtw)
    torch.cuda.synchronize()
    assert bool((cx[::2] == 0).all()) and bool((cw[::2] == 0).all())
    assert not bool(torch.signbit(cx[::2]).any())


# --------------------------------------------------------------------------- FP8
def _exhaustive_bf16_rows(H=7168):
    """Every finite bf16 pattern, in 128-channel groups that each hold one
    448: the plain and the power-of-two scales are then exactly 1, so the
    codes are the E4M3 encodings of the bf16 values themselves."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (pats.astype(np.uint32) << 16).view(np.float32)
    pats = pats[np.isfinite(f) & (np.abs(f) <= 448.0)]
    per = 127
    ngroups = -(-pats.size // per)
    groups = np.zeros((ngroups, 128), np.uint16)
    flat = np.zeros(ngroups * per, np.uint16)
    flat[:pats.size] = pats
    groups[:, :per] = flat.reshape(ngroups, per)
    groups[:, per] = 0x43E0                # 448.0 in bf16
    G = H // 128
    rows = -(-ngroups // G)
    out = np.zeros((rows * G, 128), np.uint16)
    out[:, 127] = 0x43E0
    out[:ngroups] = groups
    return out.reshape(rows, H)


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_cast_exhaustive_bf16(round_scale):
    say("fp8 cast exhaustive bf16", round_scale)
    xb = _exhaustive_bf16_rows()
    N, H = xb.shape
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    idx = torch.zeros((N, 1), dtype=torch.int64)          # every token to expert 0 on rank 0
    xd, idxd = x.to(DEV), idx.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, 1, 1, 1)
    rx, rs, _, _, _, h = miep.dispatch(xd, idxd, None, ntpr, itr, ntpe, 1, 1, cast_to_fp8=True,
                                       round_scale=round_scale)
    codes, sci, _ = oracle.fp8_quantize(xb, round_scale)
    assert np.array_equal(npy(rs).view(np.uint32), sci.view(np.uint32))
    assert np.all(sci == 1.0)
    got = u8(rx)
    bad = np.nonzero(got != codes)
    assert bad[0].size == 0, (xb[bad][:8], got[bad][:8], codes[bad][:8])


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_cast_random_magnitudes(round_scale):
    """14.7M scaled products: rows and 128-channel groups spanning 1e-8 .. 1e4,
    some groups with one dominant outlier, every code and scale compared."""
    say("fp8 cast random magnitudes", round_scale)
    N, H = 2048, 7168
    g = torch.Generator().manual_seed(21)
    x = torch.randn((N, H), generator=g)
    G = H // 128
    mag = 10.0 ** (torch.rand((N, G), generator=g) * 12 - 8)
    x = (x.view(N, G, 128) * mag.unsqueeze(2))
    out = torch.rand((N, G), generator=g) < 0.2
    x[:, :, 0] = torch.where(out, x[:, :, 0] * 1000.0, x[:, :, 0])
    x = x.view(N, H).to(torch.bfloat16)
    xb = wl.bf16_bits(x)
    idx = torch.zeros((N, 1), dtype=torch.int64)
    xd, idxd = x.to(DEV), idx.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, 1, 1, 1)
    rx, rs, _, _, _, h = miep.dispatch(xd, idxd, None, ntpr, itr, ntpe, 1, 1, cast_to_fp8=True,
                                       round_scale=round_scale)
    codes, sci, _ = oracle.fp8_quantize(xb, round_scale)
    assert np.array_equal(npy(rs).view(np.uint32), sci.view(np.uint32))
    got = u8(rx)
    bad = np.nonzero(got != codes)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], codes[bad][:5])


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_dispatch_kinds_small(round_scale):
    """Fused cast and pre-quantised FP8 dispatch on a ragged multi-tile case,
    with magnitudes that exercise subnormal codes and saturation edges."""
    w = _small_workload("fp8", 3, 200, 1152, 48, 16, 4, 5, 1)
    say("fp8 kinds", w, round_scale)
    x, idx, wts = _inputs(w, 8)
    scale = torch.tensor(np.random.default_rng(0).choice([1e-6, 1e-3, 1.0, 300.0, 3e4], (w.N, 1)),
                         dtype=torch.float32)
    x = (x.float() * scale).to(torch.bfloat16)
    x[5, :128] = 0.0
    xb = wl.bf16_bits(x)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    ref_lay = oracle.layout(idx.numpy(), w.S, w.E, w.R)
    ref = _ref_dispatch(w, xb, idx.numpy(), wts.numpy(), ref_lay, x_kind=oracle.X_BF16_CAST_FP8,
                        round_scale=round_scale)
    out = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, cast_to_fp8=True, round_scale=round_scale,
                        use_ue8m0=round_scale)
    rx, rs, rti, rtw, _, h = out[:6]
    torch.cuda.synchronize()
    _check_handle(h, ref)
    assert np.array_equal(u8(rx), ref["recv_x"])
    assert np.array_equal(npy(rs).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
    if round_scale:
        # UE8M0 exponent bytes against the oracle's (fresh and cached dispatch)
        ref_ue = _ref_dispatch(w, xb, idx.numpy(), wts.numpy(), ref_lay, x_kind=oracle.X_BF16_CAST_FP8,
                               round_scale=True, use_ue8m0=True)["recv_x_scales_ue8m0"]
        assert np.array_equal(npy(out[6]), ref_ue)
        _, _, cue = miep.cached_dispatch(xd, h, cast_to_fp8=True, round_scale=True, use_ue8m0=True)
        assert np.array_equal(npy(cue), ref_ue)
    # pre-quantised codes + scales travel unchanged
    codes, sci, _ = oracle.fp8_quantize(xb, round_scale)
    cd = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(DEV)
    rx2, rs2 = miep.cached_dispatch(cd, h, x_scales=torch.from_numpy(sci).to(DEV))
    assert np.array_equal(u8(rx2), ref["recv_x"])
    assert np.array_equal(npy(rs2).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
    # cached dispatch with the fused cast reproduces the fresh result
    rx3, rs3 = miep.cached_dispatch(xd, h, cast_to_fp8=True, round_scale=round_scale)
    assert torch.equal(rx3.view(torch.uint8), rx.view(torch.uint8)) and torch.equal(rs3, rs)


@pytest.mark.parametrize("round_scale", [False, True])
def test_large_two_level_fp8_roundtrip(round_scale):
    """Large workload: 16384 tokens, 64 ranks in 8 RDMA groups, FP8-cast
    dispatch, bf16 combine of the dequantised identity experts.  Everything is
    compared in full: layout, handle, every receive row's E4M3 codes and fp32
    scales, the top-k metadata, and the combine (bit-exact against the
    oracle, max relative error < 1e-2 against its fp32 sums, calc_diff < 5e-6
    for the identity round trip).

    The oracle's fused-cast dispatch quantises once per receive row; here it
    quantises each source row once (threads over row chunks) and dispatches
    the codes as pre-quantised FP8, which the CPU pins show to be the same
    result (the cast is a function of the source row alone)."""
    w = wl.LARGE
    say("large fp8", round_scale)
    x, idx, wts = _inputs(w, 0)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    lay = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    ref_lay = _check_layout(w, idx, lay)
    ntpr, _, ntpe, itr = lay
    out = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C, cast_to_fp8=True, round_scale=round_scale,
                        use_ue8m0=round_scale)
    rx, rs, rti, rtw, nrte, h = out[:6]
    xb = wl.bf16_bits(x)
    codes, sci, ue = oracle.fp8_quantize(xb, round_scale, threads=16)
    ref = oracle.dispatch(codes, idx.numpy(), wts.numpy(), ref_lay["is_token_in_rank"],
                          ref_lay["num_tokens_per_expert"], S=w.S, E=w.E, R=w.R, C=w.C, x_kind=oracle.X_FP8,
                          x_scales=sci)
    torch.cuda.synchronize()
    _check_handle(h, ref)
    assert h.recv_capacity == ref["num_recv"]
    assert np.array_equal(u8(rx), ref["recv_x"])
    assert np.array_equal(npy(rs).view(np.uint32), ref["recv_x_scales"].view(np.uint32))
    assert np.array_equal(npy(rti), ref["recv_topk_idx"])
    assert np.array_equal(npy(rtw).view(np.uint32), ref["recv_topk_weights"].view(np.uint32))
    assert np.array_equal(npy(nrte), ref["num_recv_tokens_per_expert"])
    if round_scale:
        # exponent bytes: the oracle's per-source bytes, placed by the oracle's own send_head
        rows = ref["recv_rank_offset"][:-1][None, :] + ref["send_head"]
        n_of_row = np.empty(ref["num_recv"], np.int64)
        sel = ref["send_head"] >= 0
        n_of_row[rows[sel]] = np.nonzero(sel)[0]
        assert np.array_equal(npy(out[6]), ue[n_of_row])
    # identity experts on the oracle's dequantised receive rows, bf16 combine
    ref_rx = torch.from_numpy(ref["recv_x"]).view(torch.float8_e4m3fn)
    ref_rs = torch.from_numpy(ref["recv_x_scales"])
    y = (ref_rx.float() * ref_rs.repeat_interleave(128, dim=1)).to(torch.bfloat16)
    del ref_rx
    cx, cw = miep.combine(y.to(DEV), h, rtw)
    rc = oracle.combine(wl.bf16_bits(y), ref["recv_topk_weights"], ref["send_head"], ref["recv_rank_offset"], S=w.S,
                        want_f32=True)
    del y
    got = u16(cx)
    assert np.array_equal(got, rc["combined_x"])
    assert np.array_equal(npy(cw).view(np.uint32), rc["combined_topk_weights"].view(np.uint32))
    g = oracle.bf16_to_f32(got).reshape(got.shape).astype(np.float64)
    f = rc["combined_f32"].astype(np.float64)
    assert (np.abs(g - f) / np.maximum(np.abs(f), 1e-6)).max() < 1e-2
    deq = (torch.from_numpy(codes).view(torch.float8_e4m3fn).float() *
           torch.from_numpy(sci).repeat_interleave(128, dim=1)).to(torch.bfloat16).float().numpy().astype(np.float64)
    cnt = ref_lay["is_token_in_rank"].sum(axis=1).astype(np.float64)
    ok = cnt > 0
    assert oracle.calc_diff(g[ok] / cnt[ok, None], deq[ok]) < 5e-6
    assert np.all(g[~ok] == 0)
    valid = (idx.numpy() >= 0) & ok[:, None]
    assert np.array_equal(npy(cw)[valid], wts.numpy()[valid])


# --------------------------------------------------------------------------- low-latency
def _check_ll(out, ref, use_fp8, use_ue8m0, L, S, M):
    cnt = ref["msg_count"]
    assert np.array_equal(npy(out["msg_count"]), cnt)
    assert np.array_equal(npy(out["packed_recv_count"]), ref["packed_recv_count"])
    assert np.array_equal(npy(out["packed_recv_layout_range"]), ref["packed_recv_layout_range"])
    msg = u8(out["msg_buf"])
    H = ref["packed_recv_x"].shape[-1]
    used = 16 + (H + 4 * (H // 128) if use_fp8 else 2 * H)   # the stride's padding carries no value
    for l in range(L):
        for s in range(S):
            n = cnt[l, s]
            assert np.array_equal(msg[l, s, :n, :used], ref["msg_buf"][l, s, :n, :used]), (l, s)
        n = ref["packed_recv_count"][l]
        assert np.array_equal(npy(out["packed_recv_src_info"])[l, :n], ref["packed_recv_src_info"][l, :n])
        if use_fp8:
            assert np.array_equal(u8(out["packed_recv_x"][l, :n]), ref["packed_recv_x"][l, :n])
            assert np.array_equal(npy(out["packed_recv_x_scales"][l, :n]).view(np.uint32),
                                  ref["packed_recv_x_scales"][l, :n].view(np.uint32))
            if use_ue8m0:
                assert np.array_equal(npy(out["packed_recv_x_scales_ue8m0"][l, :n]),
                                      ref["packed_recv_x_scales_ue8m0"][l, :n])
        else:
            assert np.array_equal(u16(out["packed_recv_x"][l, :n]), ref["packed_recv_x"][l, :n])


LL_SMALL = [
    # name, R, T, M, H, E, K, d
    ("ll-tiny", 4, 6, 8, 512, 16, 3, 1),
    ("ll-ragged", 6, 300, 320, 1536, 24, 4, 5),
    ("ll-r72", 72, 20, 24, 512, 144, 4, 70),        # > 64 earlier sources summed for the packed range
    ("ll-fp8-wide", 4, 40, 48, 2560, 16, 4, 1),     # FP8 rows of 160 pairs: two pairs per lane, partial last slice
    ("ll-h640", 4, 20, 24, 640, 16, 4, 2),           # H % 512 != 0: FP8 messages padded to a 16-byte stride
]


@pytest.mark.parametrize("case", LL_SMALL, ids=[c[0] for c in LL_SMALL])
@pytest.mark.parametrize("flags", [(False, False, False), (True, False, False), (True, True, False),
                                   (True, True, True)], ids=["bf16", "fp8", "fp8-pow2", "fp8-ue8m0"])
def test_ll_small(case, flags):
    name, R, T, M, H, E, K, d = case
    use_fp8, round_scale, use_ue8m0 = flags
    say("ll", case, flags)
    g = torch.Generator().manual_seed(11)
    idx = wl.topk_uniform(R * T, E, K, g)
    idx[::7, 0] = -1
    if K > 1:
        idx[::5, 1] = idx[::5, 0]          # duplicated expert: two messages
    x = wl.activations(R * T, H, g)
    stats = torch.full((E // R,), 3, dtype=torch.int32)
    out = miep.low_latency_dispatch(x.to(DEV), idx.to(DEV), M, E, d, R, use_fp8, round_scale, use_ue8m0,
                                    stats.to(DEV))
    ref = oracle.ll_dispatch(wl.bf16_bits(x), idx.numpy(), S=R, M=M, E=E, R=R, dest_rank=d, use_fp8=use_fp8,
                             round_scale=round_scale, use_ue8m0=use_ue8m0, cumulative_stats=stats.numpy())
    torch.cuda.synchronize()
    _check_ll(out, ref, use_fp8, use_ue8m0, E // R, R, M)
    assert np.array_equal(npy(out["cumulative_local_expert_recv_stats"]), ref["cumulative_local_expert_recv_stats"])


@pytest.mark.parametrize("flags", [(True, False, False), (True, True, True), (False, False, False)],
                         ids=["fp8", "fp8-ue8m0", "bf16"])
def test_ll_full_workload(flags):
    w = wl.LL
    use_fp8, round_scale, use_ue8m0 = flags
    say("ll full", flags)
    inp = wl.ll_inputs(w, 0)
    out = miep.low_latency_dispatch(inp["x"].to(DEV), inp["topk_idx"].to(DEV), w.M, w.E, w.dest_rank, w.R, use_fp8,
                                    round_scale, use_ue8m0)
    ref = oracle.ll_dispatch(wl.bf16_bits(inp["x"]), inp["topk_idx"].numpy(), S=w.S, M=w.M, E=w.E, R=w.R,
                             dest_rank=w.dest_rank, use_fp8=use_fp8, round_scale=round_scale, use_ue8m0=use_ue8m0)
    torch.cuda.synchronize()
    _check_ll(out, ref, use_fp8, use_ue8m0, w.L, w.S, w.M)


def test_repeat_is_deterministic():
    w = wl.NORMAL
    say("determinism", w.name)
    x, idx, wts = _inputs(w, 0)
    xd, idxd, wd = x.to(DEV), idx.to(DEV), wts.to(DEV)
    outs = []
    for _ in range(2):
        ntpr, _, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
        recv_x, _, rti, rtw, _, h = miep.dispatch(xd, idxd, wd, ntpr, itr, ntpe, w.E, w.C)
        cx, cw = miep.combine(recv_x, h, rtw)
        outs.append((recv_x.clone(), h.send_head.clone(), cx.clone(), cw.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
