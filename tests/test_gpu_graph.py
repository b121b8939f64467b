"""HIP graph capture of the hot path: the allocation-free ``*_into`` calls are
captured on torch's capture stream and replayed several times, with eager
work and synchronisations between the replays; every replay must reproduce
the eager outputs bit for bit (no memset or copy nodes are recorded: the
library clears with its own fill kernels)."""
import sys

import numpy as np
import pytest
import torch

from combine_get_dispatch_histogram_amd import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_get_dispatch_histogram_amd as miep  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def test_normal_step_graph_replays_match_eager():
    w = wl.NORMAL
    say("graph normal step", w.name)
    inp = wl.normal_inputs(w, 0)
    x, idx, wts = inp["x"].to(DEV), inp["topk_idx"].to(DEV), inp["topk_weights"].to(DEV)
    S, R, E, K, H, N, C = w.S, w.R, w.E, w.K, w.H, w.N, w.C
    i32 = dict(dtype=torch.int32, device=DEV)
    ntpr, ntpe = torch.empty((S, R), **i32), torch.empty((S, E), **i32)
    itr = torch.empty((N, R), dtype=torch.bool, device=DEV)
    miep.get_dispatch_layout_into(idx, E, R, S, ntpr, None, ntpe, itr)
    rows = int(ntpr.sum().item())
    h = miep.Handle.allocate(itr, S, K, E, C, rows)
    recv_x = torch.empty((rows, H), dtype=torch.bfloat16, device=DEV)
    rti = torch.empty((rows, K), dtype=torch.int64, device=DEV)
    rtw = torch.empty((rows, K), dtype=torch.float32, device=DEV)
    nrte = torch.empty((R, E // R), **i32)
    y = wl.expert_outputs(rows, H, seed=1).to(DEV)
    cx = torch.empty((N, H), dtype=torch.bfloat16, device=DEV)
    cw = torch.empty((N, K), dtype=torch.float32, device=DEV)

    def step():
        miep.get_dispatch_layout_into(idx, E, R, S, ntpr, None, ntpe, itr)
        miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, None, rti, rtw, nrte)
        miep.combine_into(y, h, cx, rtw, cw)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (recv_x, rti, rtw, h.send_head, h.recv_rank_offset, nrte, cx, cw)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    scratch_y = wl.expert_outputs(rows, H, seed=2).to(DEV)
    for rep in range(3):
        for t in (recv_x, cx, cw, h.send_head):
            t.fill_(0 if t.dtype != torch.bfloat16 else 1)   # poison the outputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (recv_x, rti, rtw, h.send_head, h.recv_rank_offset, nrte, cx, cw)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d differs from eager" % rep
        # eager work between replays on the same buffers' neighbours
        other = torch.empty_like(cx)
        miep.combine_into(scratch_y, h, other, None, None)
        torch.cuda.synchronize()


def test_low_latency_graph_replays_match_eager():
    w = wl.LL
    say("graph ll", w.name)
    inp = wl.ll_inputs(w, 0)
    x, idx = inp["x"].to(DEV), inp["topk_idx"].to(DEV)
    R, M, H, E, L, K, d = w.R, w.M, w.H, w.E, w.L, w.K, w.dest_rank
    wts = wl.gate_weights(w.N, K, torch.Generator().manual_seed(1)).to(DEV)
    mb = miep.ll_msg_bytes(H, True)
    bufs = dict(msg_buf=torch.empty((L, R, M, mb), dtype=torch.uint8, device=DEV),
                msg_count=torch.empty((L, R), dtype=torch.int32, device=DEV),
                packed_recv_x=torch.empty((L, R * M, H), dtype=torch.float8_e4m3fn, device=DEV),
                packed_recv_x_scales=torch.empty((L, R * M, H // 128), dtype=torch.float32, device=DEV),
                packed_recv_x_scales_ue8m0=torch.empty((L, R * M, H // 128), dtype=torch.uint8, device=DEV),
                packed_recv_src_info=torch.empty((L, R * M), dtype=torch.int32, device=DEV),
                packed_recv_layout_range=torch.empty((L, R), dtype=torch.int64, device=DEV),
                packed_recv_count=torch.empty((L,), dtype=torch.int32, device=DEV))
    stats = torch.zeros((L,), dtype=torch.int32, device=DEV)
    mask = torch.zeros((R,), dtype=torch.int32, device=DEV)
    y = wl.expert_outputs(L * R * M, H, seed=3).view(L, R * M, H).to(DEV)
    cx = torch.empty((w.N, H), dtype=torch.bfloat16, device=DEV)

    def step():
        miep.low_latency_dispatch_into(x, idx, R, M, E, d, True, True, True, **bufs,
                                       cumulative_local_expert_recv_stats=stats, mask_buffer=mask)
        miep.low_latency_combine_into(y, idx, wts, bufs["packed_recv_src_info"], bufs["packed_recv_layout_range"],
                                      R, M, E, d, cx)

    step()
    torch.cuda.synchronize()
    count = bufs["packed_recv_count"].clone()
    keys = ("packed_recv_count", "packed_recv_layout_range", "packed_recv_src_info")
    ref = {k: bufs[k].clone() for k in keys}
    ref_cx = cx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    stats.zero_()
    torch.cuda.synchronize()
    for rep in range(3):
        cx.fill_(1)
        bufs["packed_recv_src_info"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            n = ref[k]
            got = bufs[k]
            if k == "packed_recv_src_info":
                for l in range(L):
                    c = int(count[l])
                    assert torch.equal(got[l, :c], n[l, :c]), (rep, k, l)
            else:
                assert torch.equal(got, n), (rep, k)
        assert torch.equal(cx, ref_cx), rep
        assert torch.equal(stats, count * (rep + 1)), "cumulative stats after %d replays" % (rep + 1)
        # eager work between replays: mask and unmask a rank
        miep.update_mask_buffer(mask, 3, True)
        miep.clean_mask_buffer(mask)
        torch.cuda.synchronize()
    assert np.array_equal(mask.cpu().numpy(), np.zeros(R, np.int32))
