"""Independent pure-Python brute force for tiny inputs.

Written separately from the C oracle (different data structures, exact
rational arithmetic for the encoders, library routines for IEEE rounding) so
that a mistake in one does not repeat in the other.  Slow on purpose; only
for the shapes the CPU tests feed it.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

# ----------------------------------------------------------------- E4M3FN by exact search
# OCP 8-bit floating point E4M3: value = (-1)^s 2^(e-7) (1 + m/8) for e > 0,
# (-1)^s 2^-6 (m/8) for e = 0, and S.1111.111 is NaN; no infinities.


def e4m3_value(code: int):
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


E4M3_POS = [(c, e4m3_value(c)) for c in range(0x7F)]   # all non-negative finite codes


def e4m3_encode_exact(a: float) -> int:
    """Nearest finite E4M3 value (ties to even code), by exact search over every code."""
    if math.isnan(a):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, a) < 0 else 0
    m = Fraction(abs(a))
    best = None
    for c, v in E4M3_POS:
        d = abs(m - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sign | best[1]


# ----------------------------------------------------------------- bf16 via library cast
def bf16_round_lib(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits using torch's (round-to-nearest-even) cast."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def bf16_value(bits: int) -> np.float32:
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


# ----------------------------------------------------------------- FP8 per-128 quantisation
def fp8_scales(amax: np.float32, round_scale: bool):
    amax = max(np.float32(amax), np.float32(1e-4))
    if round_scale:
        v = Fraction(float(np.float32(amax) / np.float32(448.0)))
        e = -200
        while Fraction(2) ** e < v:          # smallest power of two >= v
            e += 1
        return np.float32(2.0 ** -e), np.float32(2.0 ** e), e
    return np.float32(448.0) / np.float32(amax), np.float32(amax) / np.float32(448.0), None


def fp8_quantize_row(row_bits, round_scale: bool):
    H = len(row_bits)
    codes, scales, exps = [], [], []
    for g0 in range(0, H, 128):
        vals = [bf16_value(int(b)) for b in row_bits[g0:g0 + 128]]
        amax = np.float32(max(abs(float(v)) for v in vals))
        sc, sci, e = fp8_scales(amax, round_scale)
        for v in vals:
            codes.append(e4m3_encode_exact(float(np.float32(v) * sc)))
        scales.append(sci)
        exps.append(e)
    return codes, scales, exps


# ----------------------------------------------------------------- layout
def layout(topk_idx, S: int, E: int, R: int):
    idx = [list(map(int, row)) for row in np.asarray(topk_idx)]
    N = len(idx)
    T = N // S
    L = E // R
    per_rank = [[0] * R for _ in range(S)]
    per_expert = [[0] * E for _ in range(S)]
    G = R // 8 if R > 8 else 0
    per_rdma = [[0] * G for _ in range(S)]
    in_rank = [[0] * R for _ in range(N)]
    for n, row in enumerate(idx):
        s = n // T
        ranks = set()
        for e in row:
            if 0 <= e < E:
                per_expert[s][e] += 1
                ranks.add(e // L)
        for r in ranks:
            in_rank[n][r] = 1
            per_rank[s][r] += 1
        for g in {r // 8 for r in ranks}:
            if G:
                per_rdma[s][g] += 1
    return dict(num_tokens_per_rank=per_rank, num_tokens_per_expert=per_expert,
                num_tokens_per_rdma_rank=per_rdma if G else None, is_token_in_rank=in_rank)


# ----------------------------------------------------------------- dispatch (as lists of source tokens)
def dispatch_plan(in_rank, S: int, C: int):
    """For every rank, the ordered list of (s, t) it receives, plus the prefix matrices."""
    in_rank = np.asarray(in_rank)
    N, R = in_rank.shape
    T = N // S
    tc = -(-T // C) if T else 0
    received = {r: [] for r in range(R)}
    for s in range(S):
        for t in range(T):
            for r in range(R):
                if in_rank[s * T + t, r]:
                    received[r].append((s, t))
    cpm = np.zeros((S, R, C), np.int64)
    for s in range(S):
        for r in range(R):
            for c in range(C):
                cpm[s, r, c] = sum(1 for t in range(T) if t < (c + 1) * tc and in_rank[s * T + t, r])
    rpm = np.zeros((S, R), np.int64)
    for s in range(S):
        for r in range(R):
            rpm[s, r] = sum(1 for (s2, _t) in received[r] if s2 <= s)
    rcpm = np.zeros((R, S, C), np.int64)
    for r in range(R):
        for s in range(S):
            for c in range(C):
                rcpm[r, s, c] = sum(1 for (s2, t2) in received[r] if s2 < s or (s2 == s and t2 < (c + 1) * tc))
    return received, cpm, rpm, rcpm


# ----------------------------------------------------------------- combine (fp32 in numpy scalars)
def combine_token(rows_f32):
    """Sum a token's contributions in ascending rank order, fp32, first-term start."""
    acc = None
    for v in rows_f32:
        acc = np.float32(v) if acc is None else np.float32(acc + np.float32(v))
    return acc


# ----------------------------------------------------------------- expected ranks per token
def expected_groups_hit(E: int, K: int, G: int) -> float:
    """Expected number of distinct groups (of E/G experts each) hit by K distinct
    uniformly chosen experts: G * (1 - C(E - E/G, K) / C(E, K))."""
    return G * (1 - math.comb(E - E // G, K) / math.comb(E, K))


# ----------------------------------------------------------------- low-latency combine
def ll_combine(y_bits, src_info, layout_range, topk_idx, S, M, E, R, d, weights=None):
    """For each source token, walk its top-k entries on rank d's experts in k order; the entry's row is
    found by scanning the (expert, source) block for rows naming the token (its occurrence among the
    token's entries for that expert picks among duplicates); fp32 sum from the first contribution."""
    L = E // R
    N, K = topk_idx.shape
    T = N // S
    H = y_bits.shape[2]
    out = np.zeros((N, H), np.float32)
    have = np.zeros(N, bool)
    for s in range(S):
        for t in range(T):
            n = s * T + t
            acc = None
            seen = {}
            for k in range(K):
                e = int(topk_idx[n, k])
                if not (d * L <= e < (d + 1) * L):
                    continue
                l = e - d * L
                occ = seen.get(e, 0)
                seen[e] = occ + 1
                begin, cnt = int(layout_range[l, s]) >> 32, int(layout_range[l, s]) & 0xFFFFFFFF
                rows = [begin + i for i in range(cnt) if src_info[l, begin + i] == t]
                if occ >= len(rows):
                    continue
                row = rows[occ]
                v = (y_bits[l, row].astype(np.uint32) << 16).view(np.float32)
                if weights is not None:
                    v = (v * np.float32(weights[n, k])).astype(np.float32)
                acc = v.copy() if acc is None else (acc + v).astype(np.float32)
            if acc is not None:
                out[n] = acc
                have[n] = True
    return out, have


# ----------------------------------------------------------------- two-level relay
def relay_plan(in_rank, S: int):
    """Group buffers of the relay: for every group of 8 ranks, the ordered list of source tokens n that
    go to any of its ranks; per RDMA row, the row it takes in each of the group's ranks (or -1)."""
    in_rank = np.asarray(in_rank)
    N, R = in_rank.shape
    G = R // 8
    rows = {g: [n for n in range(N) if any(in_rank[n, 8 * g + j] for j in range(8))] for g in range(G)}
    send_rdma_head = np.full((N, G), -1, np.int64)
    for g in range(G):
        for i, n in enumerate(rows[g]):
            send_rdma_head[n, g] = i
    nvl = {}
    for g in range(G):
        taken = [0] * 8
        for i, n in enumerate(rows[g]):
            heads = []
            for j in range(8):
                if in_rank[n, 8 * g + j]:
                    heads.append(taken[j])
                    taken[j] += 1
                else:
                    heads.append(-1)
            nvl[(g, i)] = heads
    return rows, send_rdma_head, nvl


def relay_combine(y_bits, recv_rank_offset, rows, send_rdma_head, nvl, S: int, partial_f32: bool = False):
    """Two-level sum: per group row, fp32 over the group's ranks then one bf16 rounding (torch's cast), or
    no rounding with ``partial_f32``; per token, fp32 over its groups' partials, then bf16."""
    N, G = send_rdma_head.shape
    H = y_bits.shape[1]
    partial = {}
    for g in range(G):
        for i, n in enumerate(rows[g]):
            acc = None
            for j, h in enumerate(nvl[(g, i)]):
                if h < 0:
                    continue
                v = (y_bits[int(recv_rank_offset[8 * g + j]) + h].astype(np.uint32) << 16).view(np.float32)
                acc = v.copy() if acc is None else (acc + v).astype(np.float32)
            if partial_f32:
                partial[(g, i)] = np.zeros(H, np.float32) if acc is None else acc
            else:
                partial[(g, i)] = np.zeros(H, np.uint16) if acc is None else bf16_round_lib(acc)
    out = np.zeros((N, H), np.uint16)
    for n in range(N):
        acc = None
        for g in range(G):
            i = int(send_rdma_head[n, g])
            if i < 0:
                continue
            p = partial[(g, i)]
            v = p if partial_f32 else (p.astype(np.uint32) << 16).view(np.float32)
            acc = v.copy() if acc is None else (acc + v).astype(np.float32)
        if acc is not None:
            out[n] = bf16_round_lib(acc)
    return out, partial
