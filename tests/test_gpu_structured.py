"""Placement checked without the oracle: every token row carries its own
(source, token) in exact bf16 integers, so each rank's received rows can be
read back and compared with the routing directly (the pages' structured-input
kind beside the pure-random one), for the direct dispatch, the relay and the
low-latency dispatch."""
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


def _decode(rows):
    r = rows.float().cpu().numpy()
    assert np.all(r[:, 0::3] == r[:, :1]) and np.all(r[:, 1::3] == r[:, 1:2]) and np.all(r[:, 2::3] == r[:, 2:3])
    return r[:, 0].astype(np.int64), (r[:, 1] + 256 * r[:, 2]).astype(np.int64)


@pytest.mark.parametrize("wname,path", [("tiny", "direct"), ("normal", "direct"), ("large", "direct"),
                                        ("large", "relay")])      # the relay needs more than 8 ranks
def test_structured_placement(wname, path):
    w = wl.WORKLOADS[wname]
    say("structured", wname, path)
    idx = wl.normal_inputs(w, 0)["topk_idx"]
    x = wl.structured_x(w.S, w.T, w.H)
    idxd = idx.to(DEV)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idxd, w.E, w.R, w.S)
    if path == "direct":
        recv_x, _, rti, _, _, h = miep.dispatch(x.to(DEV), idxd, None, ntpr, itr, ntpe, w.E, w.C)
    else:
        recv_x, _, rti, _, _, h, rh, _, _ = miep.relay_dispatch(x.to(DEV), idxd, None, ntpr, ntp_rdma, itr, ntpe,
                                                               w.E, w.C)
    off = h.recv_rank_offset.cpu().numpy()
    src, tok = _decode(recv_x)
    assert np.array_equal(tok, h.recv_src_idx.cpu().numpy())
    member = itr.cpu().numpy()
    L = w.E // w.R
    idx_np = idx.numpy()
    for r in range(w.R):
        want = [(n // w.T, n % w.T) for n in np.nonzero(member[:, r])[0]]   # (source, token) ascending
        got = list(zip(src[off[r]:off[r + 1]].tolist(), tok[off[r]:off[r + 1]].tolist()))
        assert got == want, r
        # the local expert ids a row carries are the token's entries on this rank
        for q, (s, t) in enumerate(got[:64]):
            e = idx_np[s * w.T + t]
            mine = (e >= 0) & (e // L == r)
            assert np.array_equal(rti[off[r] + q].cpu().numpy(), np.where(mine, e - r * L, -1))
    # identity combine: each token comes back times its number of receiving ranks
    cx, _ = (miep.combine(recv_x, h) if path == "direct" else miep.relay_combine(recv_x, h, rh))
    cnt = member.sum(axis=1)
    got = cx.float().cpu().numpy()
    want = x.float().numpy() * cnt[:, None]
    exact = cnt > 0
    small = want.max(axis=1) <= 256                  # products that stay exact in bf16
    assert np.array_equal(got[exact & small], want[exact & small])


def test_structured_low_latency():
    w = wl.LL
    say("structured ll", w.name)
    idx = wl.ll_inputs(w, 0)["topk_idx"]
    x = wl.structured_x(w.S, w.T, w.H)
    out = miep.low_latency_dispatch(x.to(DEV), idx.to(DEV), w.M, w.E, w.dest_rank, w.R, False)
    lr = out["packed_recv_layout_range"].cpu().numpy()
    idx_np = idx.numpy()
    for l in range(w.L):
        e = w.dest_rank * w.L + l
        for s in range(w.S):
            begin, cnt = int(lr[l, s]) >> 32, int(lr[l, s]) & 0xFFFFFFFF
            rows = out["packed_recv_x"][l, begin:begin + cnt]
            src, tok = _decode(rows) if cnt else (np.zeros(0, np.int64), np.zeros(0, np.int64))
            want = [t for t in range(w.T) for k in range(w.K) if idx_np[s * w.T + t, k] == e][:w.M]
            assert np.all(src == s)
            assert tok.tolist() == want, (l, s)
