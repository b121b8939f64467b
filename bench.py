#!/usr/bin/env python3
"""Throughput of the MoE expert-parallel core on one MI355X.

Headline workload ("normal"): 4096 tokens as 8 source partitions of 512,
hidden 7168 bf16, 256 experts on 8 logical ranks, top-8, 24 channels.  One
step = get_dispatch_layout -> dispatch (notify + pack) -> combine of
synthetic expert outputs, all inputs resident in HBM.  The JSON line reports
tokens/s for the whole step, the HBM roofline of the dominant kernel (HIP
events on the stream the kernels run on), the other hot-path stages measured
separately (cached dispatch, FP8 low-latency dispatch, the large FP8
two-level workload, the skewed workload) and the CPU oracle timed on the host.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")


# --------------------------------------------------------------------------- algorithmic bytes
# Bytes each kernel must move at minimum (every input read once, every output
# written once), per launch.  rows = receive rows written (sum over tokens of
# the number of ranks that receive the token).
def bytes_layout(N, K, R, E, S):
    G = R // 8 if R > 8 else 0
    return N * K * 8 + N * R + S * (R + E + G) * 4


def bytes_notify(N, R, S, C, E):
    return N * R + N * R * 4 + S * R * 4 + 2 * S * R * C * 4 + (R + 1) * 4 + S * E * 4 + E * 4


def bytes_pack(N, H, K, R, rows, kind="bf16", meta=True):
    row_in = 2 * H if kind in ("bf16", "cast") else H
    row_out = 2 * H if kind == "bf16" else H + 4 * (H // 128)
    b = N * row_in + N * R * 4 + rows * row_out
    if kind == "fp8":
        b += N * 4 * (H // 128)
    if meta:
        b += N * K * 12 + rows * (4 + 12 * K)
    return b


def bytes_combine(N, H, K, R, rows, weights=True):
    b = N * R * 4 + rows * 2 * H + N * 2 * H
    if weights:
        b += rows * 4 * K + N * 4 * K
    return b


def bytes_ll(msgs, distinct_tokens, H, use_fp8, R, L):
    """Low-latency dispatch: each distinct token's row read, every message
    written once, and its packed row (payload, scales, source index) written
    once; plus the per-block counts and layout ranges."""
    mb = 16 + (H + 4 * (H // 128) if use_fp8 else 2 * H)
    pb = mb - 16
    return distinct_tokens * 2 * H + msgs * mb + msgs * (pb + 4) + L * R * (4 + 8)


def bytes_ll_combine(msgs, N, H, K, weighted):
    """Low-latency combine: every packed row read once (and its src_info), every
    token's top-k row (and weights) read and its combined row written."""
    return msgs * (2 * H + 4) + N * (2 * H + K * (8 + (4 if weighted else 0)))


def bytes_relay_dispatch(N, H, K, R, S, C, E, rows, grows, kind="cast"):
    """Relay dispatch: the ranks' notify and the groups' notify, the first hop
    (x read once, one row per (token, group)), the bookkeeping (8 heads per
    group row) and the second hop (each group row read once and written to
    its ranks with the top-k metadata of its source token)."""
    G = R // 8
    row_in = 2 * H if kind in ("bf16", "cast") else H
    row_out = 2 * H if kind == "bf16" else H + 4 * (H // 128)
    notify = bytes_notify(N, R, S, C, E) + N * R + N * G * 4 + S * G * 4 + 2 * S * G * C * 4 + (G + 1) * 4
    meta = N * G * 4 + grows * (32 + 32 + 4)   # per group row: 8 send_head entries in, 8 heads + source id out
    hop1 = N * row_in + N * G * 4 + grows * row_out
    hop2 = grows * (row_out + 32 + 4 + K * 12) + rows * (row_out + 4 + 12 * K)
    return notify + meta + hop1 + hop2


def bytes_relay_combine(N, H, K, R, rows, grows, weights=True, partial_f32=False):
    """Two-level combine: every received row read once into its group row's
    partial (written once: 2H bytes, or 4H with fp32 partials), every partial
    read once into its token's row."""
    G = R // 8
    pb = 4 if partial_f32 else 2
    b = grows * 32 + rows * 2 * H + grows * pb * H + N * G * 4 + grows * pb * H + N * 2 * H
    if weights:
        b += rows * 4 * K + 2 * grows * 4 * K + N * 4 * K
    return b


# --------------------------------------------------------------------------- helpers
def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_get_dispatch_histogram_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, kernel_src, launches_bytes_key=None):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "normal_hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kernel_key)
    if not k or k.get("src_hash") != src_hash(*kernel_src):
        return None
    return k.get("traffic_bytes_per_launch")


LEAD_CYCLES = 200000   # GPU spin ahead of a short timed call (about 0.1 ms)


class Timer:
    """HIP events recorded on the current stream around each call.

    ``lead_cycles`` > 0 first enqueues a short GPU spin (torch.cuda._sleep) so
    that the host has queued the call before the start event runs: for calls
    shorter than their host-side launch cost the interval is then device time
    rather than host overhead."""

    def __init__(self, torch, n, lead_cycles=0):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        self.i = 0
        self.lead = lead_cycles

    def __enter__(self):
        if self.lead:
            self.torch.cuda._sleep(self.lead)
        self.ev[self.i][0].record()
        return self

    def __exit__(self, *a):
        self.ev[self.i][1].record()
        self.i += 1

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.ev[:self.i]]


def time_batched(torch, fn, iters, batch=16, warm=5):
    """Device time per call of a short call: ``batch`` calls back to back
    between two events, behind a GPU spin long enough for the host to queue
    them all, so neither host launch cost nor event overhead enters the
    per-call figure; median over ``iters`` batches, in ms."""
    for _ in range(warm):
        fn()
    t = Timer(torch, iters, LEAD_CYCLES * batch)
    for _ in range(iters):
        with t:
            for _ in range(batch):
                fn()
    torch.cuda.synchronize()
    return med(t.ms()) / batch


def pct(xs, q):
    s = sorted(xs)
    return s[min(len(s) - 1, int(q * (len(s) - 1) + 0.5))] if s else float("nan")


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2] if s else float("nan")


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


# --------------------------------------------------------------------------- GPU legs
def run_normal(torch, miep, wl, steps, warmup, only=None):
    """The normal step.  only="warm": just the warm-up and timed step loop;
    only="cold": just the cold-cache runs (for counter runs that must not mix
    the two)."""
    w = wl.NORMAL
    dev = torch.device("cuda:0")
    inp = wl.normal_inputs(w, 0)
    x = inp["x"].to(dev)
    idx = inp["topk_idx"].to(dev)
    wts = inp["topk_weights"].to(dev)
    S, R, E, K, H, N, C = w.S, w.R, w.E, w.K, w.H, w.N, w.C
    i32 = dict(dtype=torch.int32, device=dev)
    ntpr = torch.empty((S, R), **i32)
    ntpe = torch.empty((S, E), **i32)
    itr = torch.empty((N, R), dtype=torch.bool, device=dev)
    miep.get_dispatch_layout_into(idx, E, R, S, ntpr, None, ntpe, itr)
    rows = int(ntpr.sum().item())              # exact receive size (routing is fixed across steps)
    h = miep.Handle.allocate(itr, S, K, E, C, rows)
    recv_x = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    rti = torch.empty((rows, K), dtype=torch.int64, device=dev)
    rtw = torch.empty((rows, K), dtype=torch.float32, device=dev)
    nrte = torch.empty((R, E // R), **i32)
    y = wl.expert_outputs(rows, H, seed=1).to(dev)   # synthetic expert outputs in the receive layout
    cx = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    cw = torch.empty((N, K), dtype=torch.float32, device=dev)

    def step(tl=None, td=None, tc=None):
        if tl:
            with tl:
                miep.get_dispatch_layout_into(idx, E, R, S, ntpr, None, ntpe, itr)
            with td:
                miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, None, rti, rtw, nrte)
            with tc:
                miep.combine_into(y, h, cx, rtw, cw)
        else:
            miep.get_dispatch_layout_into(idx, E, R, S, ntpr, None, ntpe, itr)
            miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, None, rti, rtw, nrte)
            miep.combine_into(y, h, cx, rtw, cw)

    if only == "cold":
        return dict(cold=measure_cold(torch, dev, {
            "dispatch": lambda: miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, None, rti, rtw, nrte),
            "combine": lambda: miep.combine_into(y, h, cx, rtw, cw)}, steps))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # (1) the timed region: exactly `steps` steps, no events inside
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if only == "warm":
        return dict(wall=wall)
    # (2) the same steps again with HIP events around every call
    tl, td, tc = Timer(torch, steps), Timer(torch, steps), Timer(torch, steps)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(tl, td, tc)
    torch.cuda.synchronize()
    # (3) cached dispatch on the same handle (the pack kernel alone)
    tcd = Timer(torch, steps)
    for _ in range(steps):
        with tcd:
            miep.cached_dispatch_into(x, h, recv_x)
    torch.cuda.synchronize()
    # (4) per-launch device time of the two big kernels for the roofline: 16
    # launches back to back between two events on the launch stream
    it = max(3, min(steps, 10))
    combine_launch_ms = time_batched(torch, lambda: miep.combine_into(y, h, cx, rtw, cw), it)
    pack_launch_ms = time_batched(torch, lambda: miep.cached_dispatch_into(x, h, recv_x), it)
    # (6) the same step captured once in a HIP graph and replayed `steps` times
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - t0
    del graph
    # ... and ten steps captured in one graph (a caller capturing its loop):
    # the runtime's gap between graph launches is paid once per ten steps
    graph10 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph10):
        for _ in range(10):
            step()
    for _ in range(2):
        graph10.replay()
    torch.cuda.synchronize()
    reps10 = max(1, steps // 10)
    t0 = time.perf_counter()
    for _ in range(reps10):
        graph10.replay()
    torch.cuda.synchronize()
    graph10_ms_per_step = (time.perf_counter() - t0) * 1e3 / (10 * reps10)
    del graph10
    # (5) cold caches
    cold = measure_cold(torch, dev, {
        "dispatch": lambda: miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, None, rti, rtw, nrte),
        "combine": lambda: miep.combine_into(y, h, cx, rtw, cw)}, max(20, steps))
    return dict(w=w, rows=rows, wall=wall, layout_ms=tl.ms(), dispatch_ms=td.ms(), combine_ms=tc.ms(),
                cached_ms=tcd.ms(), combine_launch_ms=combine_launch_ms, pack_launch_ms=pack_launch_ms,
                cold=cold, graph_wall=graph_wall, graph10_ms_per_step=graph10_ms_per_step)


FLUSH_BYTES = 1 << 30


def measure_cold(torch, dev, calls, iters):
    """Each call (and the calls back to back, "pair") timed with cold caches:
    before every timed run, 1 GiB is written and a second 1 GiB is read,
    then the device synchronises.  The write evicts L2 and the 256 MB
    last-level cache; the read sweep then replaces the flush's dirty lines by
    clean ones, so that no write-back of the flush lands in the timed run and
    every byte of the call comes from HBM.  A short GPU spin ahead of the
    start event lets the host queue the call first (no launch cost in the
    interval).  Returns {name: [ms per run]}."""
    fw = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    fr = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    names = list(calls) + ["pair"]
    out = {k: Timer(torch, iters, LEAD_CYCLES) for k in names}
    for _ in range(iters):
        for k in names:
            fw.fill_(1)
            fr.max()
            torch.cuda.synchronize()
            with out[k]:
                if k == "pair":
                    for f in calls.values():
                        f()
                else:
                    calls[k]()
            torch.cuda.synchronize()
    del fw, fr
    return {k: t.ms() for k, t in out.items()}


def run_ll(torch, miep, wl, iters):
    w = wl.LL
    dev = torch.device("cuda:0")
    inp = wl.ll_inputs(w, 0)
    x = inp["x"].to(dev)
    idx = inp["topk_idx"].to(dev)
    L, R, M, H = w.L, w.R, w.M, w.H
    out = {}
    for name, fp8, rs, ue in (("fp8", True, False, False), ("fp8_ue8m0", True, True, True)):
        mb = miep.ll_msg_bytes(H, fp8)
        bufs = dict(msg_buf=torch.empty((L, R, M, mb), dtype=torch.uint8, device=dev),
                    msg_count=torch.empty((L, R), dtype=torch.int32, device=dev),
                    packed_recv_x=torch.empty((L, R * M, H), dtype=torch.float8_e4m3fn, device=dev),
                    packed_recv_x_scales=torch.empty((L, R * M, H // 128), dtype=torch.float32, device=dev),
                    packed_recv_x_scales_ue8m0=torch.empty((L, R * M, H // 128), dtype=torch.uint8, device=dev)
                    if ue else None,
                    packed_recv_src_info=torch.empty((L, R * M), dtype=torch.int32, device=dev),
                    packed_recv_layout_range=torch.empty((L, R), dtype=torch.int64, device=dev),
                    packed_recv_count=torch.empty((L,), dtype=torch.int32, device=dev))

        def call():
            miep.low_latency_dispatch_into(x, idx, R, M, w.E, w.dest_rank, fp8, rs, ue, **bufs)

        ms = time_batched(torch, call, iters)
        msgs = int(bufs["packed_recv_count"].sum().item())
        local = (idx >= w.dest_rank * L) & (idx < (w.dest_rank + 1) * L)
        distinct = int(local.any(dim=1).sum().item())
        out[name] = dict(us=round(ms * 1e3, 2), messages=msgs, tokens=distinct,
                         tokens_per_s=round(distinct / (ms / 1e3), 1),
                         gbs=round(bytes_ll(msgs, distinct, H, fp8, R, L) / (ms / 1e3) / 1e9, 1))

    # low-latency combine of bf16 expert outputs in the packed layout, gate-weighted
    y = wl.expert_outputs(L * R * M, H, seed=1).view(L, R * M, H).to(dev)
    wts = wl.gate_weights(w.N, w.K, torch.Generator().manual_seed(2)).to(dev)
    cx = torch.empty((w.N, H), dtype=torch.bfloat16, device=dev)

    def ccall():
        miep.low_latency_combine_into(y, idx, wts, bufs["packed_recv_src_info"], bufs["packed_recv_layout_range"], R, M,
                                      w.E, w.dest_rank, cx)

    ms = time_batched(torch, ccall, iters)
    out["combine"] = dict(us=round(ms * 1e3, 2), messages=msgs, tokens=w.N,
                          gbs=round(bytes_ll_combine(msgs, w.N, H, w.K, True) / (ms / 1e3) / 1e9, 1))
    return out


def run_normal_variant(torch, miep, wl, w, iters, cast_fp8):
    dev = torch.device("cuda:0")
    inp = wl.normal_inputs(w, 0)
    x = inp["x"].to(dev)
    idx = inp["topk_idx"].to(dev)
    wts = inp["topk_weights"].to(dev)
    lay = miep.get_dispatch_layout(idx, w.E, w.R, w.S)
    ntpr, ntp_rdma, ntpe, itr = lay
    recv_x, recv_s, rti, rtw, nrte, h = miep.dispatch(x, idx, wts, ntpr, itr, ntpe, w.E, w.C, cast_to_fp8=cast_fp8)
    rows = h.recv_capacity
    if cast_fp8:
        y = (recv_x.float() * recv_s.repeat_interleave(128, dim=1)).to(torch.bfloat16)
    else:
        y = wl.expert_outputs(rows, w.H, seed=1).to(dev)
    cx = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)
    cw = torch.empty((w.N, w.K), dtype=torch.float32, device=dev)
    for _ in range(3):
        miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, recv_s, rti, rtw, nrte, cast_to_fp8=cast_fp8)
        miep.combine_into(y, h, cx, rtw, cw)
    # each call timed on its own, a few launches back to back (so the
    # write-back of one call's output does not land in another call's time)
    d_ms = time_batched(torch, lambda: miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, recv_s, rti, rtw, nrte,
                                                          cast_to_fp8=cast_fp8), iters, batch=4)
    c_ms = time_batched(torch, lambda: miep.combine_into(y, h, cx, rtw, cw), iters, batch=4)
    cd_ms = time_batched(torch, lambda: miep.cached_dispatch_into(x, h, recv_x, recv_s, cast_to_fp8=cast_fp8), iters,
                         batch=4)
    lay_ms = time_batched(torch, lambda: miep.get_dispatch_layout_into(idx, w.E, w.R, w.S, ntpr, ntp_rdma, ntpe, itr),
                          iters)
    kind = "cast" if cast_fp8 else "bf16"
    db = bytes_notify(w.N, w.R, w.S, w.C, w.E) + bytes_pack(w.N, w.H, w.K, w.R, rows, kind)
    cb = bytes_combine(w.N, w.H, w.K, w.R, rows)
    return dict(rows=rows, rho=round(rows / w.N, 4), layout_us=round(lay_ms * 1e3, 2), dispatch_us=round(d_ms * 1e3, 1),
                combine_us=round(c_ms * 1e3, 1), cached_dispatch_us=round(cd_ms * 1e3, 1),
                tokens_per_s=round(w.N / ((d_ms + c_ms) / 1e3), 1),
                dispatch_gbs=round(db / (d_ms / 1e3) / 1e9, 1), combine_gbs=round(cb / (c_ms / 1e3) / 1e9, 1),
                cached_dispatch_gbs=round(bytes_pack(w.N, w.H, w.K, w.R, rows, kind, meta=False) / (cd_ms / 1e3) / 1e9,
                                          1))


def run_relay(torch, miep, wl, iters):
    """The 64-rank workload (8 groups of 8 ranks) with the FP8 cast: relay
    dispatch and two-level combine against the direct dispatch and combine on
    the same routing (the relay's extra hop is its cost on one GPU)."""
    w = wl.LARGE
    dev = torch.device("cuda:0")
    inp = wl.normal_inputs(w, 0)
    x = inp["x"].to(dev)
    idx = inp["topk_idx"].to(dev)
    wts = inp["topk_weights"].to(dev)
    ntpr, ntp_rdma, ntpe, itr = miep.get_dispatch_layout(idx, w.E, w.R, w.S)
    recv_x, recv_s, rti, rtw, nrte, h, rh, rdma_x, rdma_s = miep.relay_dispatch(
        x, idx, wts, ntpr, ntp_rdma, itr, ntpe, w.E, w.C, cast_to_fp8=True)
    rows, grows = h.recv_capacity, rh.rdma_capacity
    y = (recv_x.float() * recv_s.repeat_interleave(128, dim=1)).to(torch.bfloat16)
    rdma_y = torch.empty((grows, w.H), dtype=torch.bfloat16, device=dev)
    rdma_w = torch.empty((grows, w.K), dtype=torch.float32, device=dev)
    cx = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)
    cw = torch.empty((w.N, w.K), dtype=torch.float32, device=dev)

    def rd():
        miep.relay_dispatch_into(x, idx, wts, ntpr, ntp_rdma, ntpe, h, rh, rdma_x, recv_x, rdma_s, recv_s, rti, rtw,
                                 nrte, cast_to_fp8=True)

    def rc():
        miep.relay_combine_into(y, h, rh, rdma_y, cx, rtw, rdma_w, cw)

    rdma_y32 = torch.empty((grows, w.H), dtype=torch.float32, device=dev)

    def rc32():                                   # fp32 group partials (rounded once)
        miep.relay_combine_into(y, h, rh, rdma_y32, cx, rtw, rdma_w, cw)

    def dd():
        miep.dispatch_into(x, idx, wts, ntpr, ntpe, h, recv_x, recv_s, rti, rtw, nrte, cast_to_fp8=True)

    def dc():
        miep.combine_into(y, h, cx, rtw, cw)

    t = {k: time_batched(torch, f, iters, batch=4) for k, f in
         (("relay_dispatch", rd), ("relay_combine", rc), ("relay_combine_f32", rc32), ("direct_dispatch", dd),
          ("direct_combine", dc))}
    bd = bytes_relay_dispatch(w.N, w.H, w.K, w.R, w.S, w.C, w.E, rows, grows)
    bc = bytes_relay_combine(w.N, w.H, w.K, w.R, rows, grows)
    return dict(rows=rows, group_rows=grows, groups_per_token=round(grows / w.N, 4),
                relay_dispatch_us=round(t["relay_dispatch"] * 1e3, 1),
                relay_combine_us=round(t["relay_combine"] * 1e3, 1),
                relay_combine_f32_partials_us=round(t["relay_combine_f32"] * 1e3, 1),
                direct_dispatch_us=round(t["direct_dispatch"] * 1e3, 1),
                direct_combine_us=round(t["direct_combine"] * 1e3, 1),
                relay_tokens_per_s=round(w.N / ((t["relay_dispatch"] + t["relay_combine"]) / 1e3), 1),
                relay_dispatch_gbs=round(bd / (t["relay_dispatch"] / 1e3) / 1e9, 1),
                relay_combine_gbs=round(bc / (t["relay_combine"] / 1e3) / 1e9, 1),
                relay_combine_f32_partials_gbs=round(
                    bytes_relay_combine(w.N, w.H, w.K, w.R, rows, grows, partial_f32=True) /
                    (t["relay_combine_f32"] / 1e3) / 1e9, 1))


def cold_summary(cold, N, nbytes):
    """Per cold-timed call: p10/p50/p90 in us, and at the median tokens/s,
    GB/s of algorithmic bytes and the fraction of the HBM peak; plus the sum
    of the separately timed dispatch and combine medians."""
    out = {}
    for k, ms in cold.items():
        m = med(ms)
        gbs = nbytes[k] / (m / 1e3) / 1e9
        out[k] = {"us_p10_p50_p90": [round(pct(ms, q) * 1e3, 2) for q in (0.1, 0.5, 0.9)],
                  "tokens_per_s": round(N / (m / 1e3), 1), "gbs": round(gbs, 1),
                  "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    t = med(cold["dispatch"]) + med(cold["combine"])
    gbs = (nbytes["dispatch"] + nbytes["combine"]) / (t / 1e3) / 1e9
    out["dispatch_plus_combine"] = {"us": round(t * 1e3, 2), "tokens_per_s": round(N / (t / 1e3), 1),
                                    "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    out["protocol"] = ("before every run: 1 GiB written, a second 1 GiB read, device synchronised; "
                       "%d runs per call; pair = dispatch and combine back to back in one timed run" % len(cold["pair"]))
    return out


# --------------------------------------------------------------------------- CPU oracle leg
def _oracle_pass(oracle, w, x, idx, wts, y):
    """One pass of the oracle over the normal workload: layout, dispatch, combine."""
    lay = oracle.layout(idx, w.S, w.E, w.R)
    d = oracle.dispatch(x, idx, wts, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=w.S, E=w.E, R=w.R,
                        C=w.C)
    oracle.combine(y, d["recv_topk_weights"], d["send_head"], d["recv_rank_offset"], S=w.S)
    return d


def _oracle_parallel_pass(oracle, w, x, idx, wts, y, pool):
    """One pass of the same oracle over the normal workload, split over the
    host cores: every piece is a call of the unchanged oracle functions on an
    independent part of the problem.
      layout:   one call per source partition (the counts of a source depend
                on its own tokens only);
      dispatch: one call per destination rank r, as a one-rank problem: the
                column r of is_token_in_rank, the top-k entries of r's experts
                renumbered to 0..L-1 (all others masked) and r's per-expert
                counts; its rows are exactly rank r's receive block;
      combine:  one call per chunk of source tokens (a token's sum reads only
                its own send_head row and the receive offsets).
    Returns the pieces the single pass returns, for the equality check."""
    import numpy as np
    S, E, R, C = w.S, w.E, w.R, w.C
    N, K = idx.shape
    T = N // S
    L = E // R
    lay = list(pool.map(lambda s: oracle.layout(idx[s * T:(s + 1) * T], 1, E, R), range(S)))
    in_rank = np.concatenate([d["is_token_in_rank"] for d in lay])
    ntpr = np.concatenate([d["num_tokens_per_rank"] for d in lay])
    ntpe = np.concatenate([d["num_tokens_per_expert"] for d in lay])

    def one_rank(r):
        lo = r * L
        mine = (idx >= lo) & (idx < lo + L)
        idx_r = np.where(mine, idx - lo, -1)
        return oracle.dispatch(x, idx_r, wts, np.ascontiguousarray(in_rank[:, r:r + 1]),
                               np.ascontiguousarray(ntpe[:, lo:lo + L]), S=S, E=L, R=1, C=C)

    parts = list(pool.map(one_rank, range(R)))
    off = np.zeros(R + 1, np.int32)
    off[1:] = np.cumsum([p["num_recv"] for p in parts])
    send_head = np.concatenate([p["send_head"] for p in parts], axis=1)
    recv_w = np.concatenate([p["recv_topk_weights"] for p in parts])
    nchunk = max(1, pool._max_workers)
    cuts = [N * i // nchunk for i in range(nchunk + 1)]

    def one_chunk(i):
        a, b = cuts[i], cuts[i + 1]
        return oracle.combine(y, recv_w, send_head[a:b], off, S=1) if b > a else None

    comb = list(pool.map(one_chunk, range(nchunk)))
    return dict(num_tokens_per_rank=ntpr, num_tokens_per_expert=ntpe, is_token_in_rank=in_rank, send_head=send_head,
                recv_rank_offset=off, recv_x=np.concatenate([p["recv_x"] for p in parts]),
                recv_topk_idx=np.concatenate([p["recv_topk_idx"] for p in parts]), recv_topk_weights=recv_w,
                combined_x=np.concatenate([c["combined_x"] for c in comb if c is not None]),
                combined_topk_weights=np.concatenate([c["combined_topk_weights"] for c in comb if c is not None]))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, budget_s, threads=None):
    """The oracle timed on the host, on the full normal workload: one
    single-threaded pass repeated for about half the budget, then the same
    pass split over the host cores (threads; capped at 16, the host share of
    one GPU) for the other half.  The reported value is the all-cores pass."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    w = wl.NORMAL
    inp = wl.normal_inputs(w, 0)
    x = wl.bf16_bits(inp["x"])
    idx = inp["topk_idx"].numpy()
    wts = inp["topk_weights"].numpy()
    lay = oracle.layout(idx, w.S, w.E, w.R)
    d = oracle.dispatch(x, idx, wts, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=w.S, E=w.E, R=w.R,
                        C=w.C)
    y = wl.bf16_bits(wl.expert_outputs(d["num_recv"], w.H, seed=1))   # input generation is not oracle work
    runs, t_total = 0, 0.0
    while runs < 1 or (t_total < budget_s / 2 and runs < 20):
        t0 = time.perf_counter()
        _oracle_pass(oracle, w, x, idx, wts, y)
        t_total += time.perf_counter() - t0
        runs += 1
    single = w.N * runs / t_total
    ncpu = os.cpu_count() or 1
    threads = threads or max(1, min(ncpu, 16))
    with ThreadPoolExecutor(threads) as pool:
        _oracle_parallel_pass(oracle, w, x, idx, wts, y, pool)      # thread start-up outside the timing
        pruns, p_total = 0, 0.0
        while pruns < 1 or (p_total < budget_s / 2 and pruns < 100):
            t0 = time.perf_counter()
            _oracle_parallel_pass(oracle, w, x, idx, wts, y, pool)
            p_total += time.perf_counter() - t0
            pruns += 1
    return dict(value=round(w.N * pruns / p_total, 1), unit="tokens/s", cores=threads, kind="oracle",
                single_thread_value=round(single, 1), cpu_count=ncpu, cpu_model=_cpu_model(),
                sample="the full normal workload (4096 tokens: layout + dispatch + combine) through the plain C "
                       "oracle (gcc -O2): one pass split over %d threads (layout per source, dispatch per "
                       "destination rank, combine per token chunk; ctypes releases the GIL), %d pass(es) in "
                       "%.1f s; single-threaded: %d pass(es) in %.1f s; the host reports %d cores"
                       % (threads, pruns, p_total, runs, t_total, ncpu))


# --------------------------------------------------------------------------- profile summaries
KERNEL_SRC = {"combine": ("combine.hip", "device.h"), "pack": ("pack.hip", "device.h"),
              "pack_cast": ("pack.hip", "device.h"), "notify": ("notify.hip", "device.h"),
              "layout": ("layout.hip", "device.h"), "ll_send": ("ll.hip", "device.h"),
              "ll_count": ("ll.hip", "device.h"), "ll_combine": ("ll.hip", "device.h")}


def _kernel_key(name):
    for k, key in (("ll_combine_kernel", "ll_combine"), ("combine_kernel", "combine"), ("pack_cast_kernel", "pack_cast"),
                   ("pack_kernel", "pack"), ("notify_chan_kernel", "notify"), ("notify_kernel", "notify"),
                   ("layout_kernel", "layout"), ("ll_send_kernel", "ll_send"), ("ll_count_src_kernel", "ll_count"),
                   ("ll_count_kernel", "ll_count"), ("relay_meta_kernel", "relay_meta")):
        if "miep::" + k in name:
            return key
    return None


def summarize_stats(stats_dir, out_md, command, title="normal workload step"):
    """rocprofv3 --kernel-trace --stats CSV -> a short markdown table of the miep kernels."""
    import csv
    import glob
    path = glob.glob(os.path.join(stats_dir, "*_kernel_stats.csv"))[0]
    lines = ["# Kernel durations: %s (rocprofv3 --kernel-trace --stats)" % title, "",
             "Command (run from the repo root on the MI355X host; `R` = repo root):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(path)):
        if "miep::" not in r["Name"]:
            continue
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f |" % (r["Name"].split("(")[0], r["Calls"],
                                                            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                                                            float(r["MaxNs"]) / 1e3))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(dirs, out_md, commands, title):
    """Any number of rocprofv3 --pmc runs -> per-kernel mean of every counter
    (per dispatch), one markdown table per run."""
    import csv
    import glob
    from collections import defaultdict
    lines = ["# Hardware counters: %s (rocprofv3 --pmc, mean per dispatch)" % title, "",
             "Commands (run from the repo root on the MI355X host; `R` = repo root):", "", "```"] + list(commands) + \
            ["```", ""]
    for d in dirs:
        agg = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(glob.glob(os.path.join(d, "*_counter_collection.csv"))[0])):
            k = _kernel_key(r["Kernel_Name"])
            if k is not None:
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        names = sorted({c for v in agg.values() for c in v})
        lines += ["| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for k in sorted(agg):
            lines.append("| %s | " % k + " | ".join("%.0f" % (sum(agg[k][c]) / len(agg[k][c])) if agg[k][c] else "-"
                                                 for c in names) + " |")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_pmc(fetch_dir, write_dir, out_json, out_md, commands, copy_mib, title="normal workload"):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each miep kernel, scaled by
    what the same counters read for the runtime's plain copy kernel of known size."""
    import csv
    import glob
    from collections import defaultdict

    def per_kernel(d, counter):
        path = glob.glob(os.path.join(d, "*_counter_collection.csv"))[0]
        vals = defaultdict(list)
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if r["Kernel_Name"] == "__amd_rocclr_copyBuffer" and v > 0:
                copy.append(v)
            k = _kernel_key(r["Kernel_Name"])
            if k:
                vals[k].append(v)
        return vals, max(copy)

    fetch, copy_f = per_kernel(fetch_dir, "FETCH_SIZE")
    write, copy_w = per_kernel(write_dir, "WRITE_SIZE")
    true_kib = copy_mib * 1024.0
    sf, sw = copy_f / true_kib, copy_w / true_kib
    out = {"copy_probe_mib": copy_mib, "fetch_scale": round(sf, 5), "write_scale": round(sw, 5),
           "commands": commands, "kernels": {}}
    lines = ["# HBM traffic per launch: %s (rocprofv3 --pmc)" % title, "",
             "Counters are KiB per dispatch.  Scale factors come from the runtime's plain copy kernel "
             "(`__amd_rocclr_copyBuffer`) of %d MiB run in the same process: FETCH_SIZE reads %.5f x its true bytes, "
             "WRITE_SIZE %.5f x." % (copy_mib, sf, sw), "", "Commands:", "", "```"] + commands + ["```", "",
             "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB (scaled) | source hash |",
             "|---|---|---|---|---|---|"]
    for k in sorted(set(fetch) & set(write)):
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write[k]) / len(write[k])
        traffic = (f / sf + w / sw) * 1024.0
        entry = {"launches": len(fetch[k]), "fetch_kib": round(f, 1), "write_kib": round(w, 1),
                 "traffic_bytes_per_launch": int(traffic)}
        if k in KERNEL_SRC:
            entry["src_hash"] = src_hash(*KERNEL_SRC[k])
        out["kernels"][k] = entry
        lines.append("| %s | %d | %.1f | %.1f | %.2f | %s |" % (k, len(fetch[k]), f, w, traffic / 1e6,
                                                               entry.get("src_hash", "-")))
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-secondary", action="store_true", help="skip the separately measured stages")
    ap.add_argument("--only-warm", action="store_true",
                    help="normal workload: only the warm-up and timed step loop (for counter runs)")
    ap.add_argument("--only-cold", action="store_true",
                    help="normal workload: only the cold-cache dispatch / combine / pair runs (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy of this many MiB first (reference for HBM counter scaling)")
    ap.add_argument("--summarize-stats", metavar="DIR", help="write profiles/ summary of a rocprofv3 --stats run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ traffic summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/<stats-name>.md: per-kernel means of any rocprofv3 --pmc runs")
    ap.add_argument("--command", action="append", default=[], help="command line(s) recorded in a summary")
    ap.add_argument("--stats-name", default="normal_step_kernels",
                    help="file name (without .md) of the --summarize-stats output under profiles/")
    ap.add_argument("--stats-title", default="normal workload step", help="workload named in that summary's title")
    ap.add_argument("--ll-only", action="store_true",
                    help="run only the low-latency dispatch and combine measurement (for a kernel profile)")
    ap.add_argument("--relay-only", action="store_true",
                    help="run only the two-level relay measurement on the 64-rank workload (for a kernel profile)")
    ap.add_argument("--workload-only", choices=("skewed", "large"),
                    help="run only the dispatch / combine / cached-dispatch measurement of one secondary workload "
                         "(for a kernel or counter profile)")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, os.path.join(PROFILES, args.stats_name + ".md"),
                        "\n".join(args.command), args.stats_title)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, os.path.join(PROFILES, args.stats_name + ".md"), args.command,
                           args.stats_title)
        return
    if args.summarize_pmc:
        name = args.stats_name if args.stats_name != "normal_step_kernels" else "normal_hbm_traffic"
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], os.path.join(PROFILES, name + ".json"),
                      os.path.join(PROFILES, name + ".md"), args.command, args.copy_probe_mib or 512,
                      args.stats_title if args.stats_title != "normal workload step" else "normal workload")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the logical ranks are partitions of one GPU's HBM and nothing here "
              "uses a second GPU (asked for --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_get_dispatch_histogram_amd as miep
    from combine_get_dispatch_histogram_amd import workloads as wl

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.ll_only:
        print(json.dumps({"ll": run_ll(torch, miep, wl, 20)}), flush=True)
        return
    if args.relay_only:
        print(json.dumps({"large_fp8_relay": run_relay(torch, miep, wl, 5)}), flush=True)
        return
    if args.only_warm or args.only_cold:
        r = run_normal(torch, miep, wl, args.steps, args.warmup, "warm" if args.only_warm else "cold")
        if args.only_warm:
            print(json.dumps({"warm_ms_per_step": round(r["wall"] * 1e3 / args.steps, 4)}), flush=True)
        else:
            print(json.dumps({"cold_us_p50": {k: round(sorted(v)[len(v) // 2] * 1e3, 2)
                                               for k, v in r["cold"].items()}}), flush=True)
        return
    if args.workload_only:
        w = wl.SKEWED if args.workload_only == "skewed" else wl.LARGE
        print(json.dumps({args.workload_only: run_normal_variant(torch, miep, wl, w, args.steps,
                                                                 args.workload_only == "large")}), flush=True)
        return

    r = run_normal(torch, miep, wl, args.steps, args.warmup)
    w, rows = r["w"], r["rows"]
    N, H, K, R, S, C, E = w.N, w.H, w.K, w.R, w.S, w.C, w.E
    ms_step = r["wall"] * 1e3 / args.steps
    lay_ms, dis_ms, com_ms, cd_ms = (mean(r[k]) for k in ("layout_ms", "dispatch_ms", "combine_ms", "cached_ms"))
    b_lay = bytes_layout(N, K, R, E, S)
    b_dis = bytes_notify(N, R, S, C, E) + bytes_pack(N, H, K, R, rows)
    b_com = bytes_combine(N, H, K, R, rows)
    b_cd = bytes_pack(N, H, K, R, rows, meta=False)
    step_bytes = b_lay + b_dis + b_com

    # dominant kernel: the combine is a single-kernel call; the pack kernel is
    # timed alone through cached dispatch (the fresh dispatch adds notify).
    cand = {"combine": (r["combine_launch_ms"], b_com, ("combine.hip", "device.h")),
            "pack": (r["pack_launch_ms"], b_cd, ("pack.hip", "device.h"))}
    dom = max(cand, key=lambda k: cand[k][0])
    d_ms, d_bytes, d_src = cand[dom]
    achieved = d_bytes / (d_ms / 1e3) / 1e9
    traffic = load_traffic(dom, d_src)
    line = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(N / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "normal", "tokens": N, "sources": S, "hidden": H, "experts": E, "ranks": R, "topk": K,
                   "channels": C, "routing": "uniform top-8 distinct", "recv_rows": rows,
                   "step": "layout + dispatch (notify + pack) + combine"},
        "achieved_gbs_step": round(step_bytes / (ms_step / 1e3) / 1e9, 1),
        "frac_of_hbm_peak_step": round(step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s_dispatch_plus_combine": round(N / ((dis_ms + com_ms) / 1e3), 1),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": d_bytes, "avg_launch_us": round(d_ms * 1e3, 2)},
        "stages_p10_p50_p90_us": {k: [round(pct(r[k + "_ms"], q) * 1e3, 2) for q in (0.1, 0.5, 0.9)]
                                  for k in ("layout", "dispatch", "combine")},
        "graph_replay_ms_per_step": round(r["graph_wall"] * 1e3 / args.steps, 4),
        "graph_replay_10_steps_ms_per_step": round(r["graph10_ms_per_step"], 4),
        "cold": cold_summary(r["cold"], N, {"dispatch": b_dis, "combine": b_com, "pair": b_dis + b_com}),
        "stages_us": {"layout": round(lay_ms * 1e3, 2), "dispatch": round(dis_ms * 1e3, 2),
                      "combine": round(com_ms * 1e3, 2), "cached_dispatch": round(cd_ms * 1e3, 2)},
        "stages_gbs": {"layout": round(b_lay / (lay_ms / 1e3) / 1e9, 1),
                       "dispatch": round(b_dis / (dis_ms / 1e3) / 1e9, 1),
                       "combine": round(b_com / (com_ms / 1e3) / 1e9, 1),
                       "cached_dispatch": round(b_cd / (cd_ms / 1e3) / 1e9, 1)},
    }
    if not args.no_secondary:
        sec = {"ll": run_ll(torch, miep, wl, 20),
               "skewed": run_normal_variant(torch, miep, wl, wl.SKEWED, 20, False),
               "large_fp8": run_normal_variant(torch, miep, wl, wl.LARGE, 10, True),
               "large_fp8_relay": run_relay(torch, miep, wl, 5)}
        line["secondary"] = sec
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
