"""CPU checks of the bench's algorithmic byte counts (the numerators of every
reported GB/s and of the roofline), against the per-unit figures the
measurement section states, worked out by hand for the normal workload
(4096 tokens, hidden 7168, top-8, 8 ranks, 256 experts, 24 channels) and
cross-checked against an independent count on a tiny routing."""
import numpy as np

import bench
import brute

N, H, K, R, E, S, C = 4096, 7168, 8, 8, 256, 8, 24
ROWS = 21626          # receive rows of the seed-0 normal routing


def test_combine_bytes_normal():
    # received rows read once (2H each), send_head read (4R per token), the
    # combined row written (2H per token), received weights read (4K per
    # row), combined weights written (4K per token)
    want = ROWS * 2 * H + N * R * 4 + N * 2 * H + ROWS * 4 * K + N * 4 * K
    assert want == 369_704_768
    assert bench.bytes_combine(N, H, K, R, ROWS) == want
    assert bench.bytes_combine(N, H, K, R, ROWS, weights=False) == want - ROWS * 4 * K - N * 4 * K


def test_pack_bytes_normal():
    # x read once, send_head read, one row written per receiving rank; a
    # fresh dispatch adds the top-k rows read (8 + 4 bytes per entry) and per
    # row the source index (4) and top-k metadata (12 per entry)
    cached = N * 2 * H + N * R * 4 + ROWS * 2 * H
    assert bench.bytes_pack(N, H, K, R, ROWS, meta=False) == cached
    assert bench.bytes_pack(N, H, K, R, ROWS) == cached + N * K * 12 + ROWS * (4 + 12 * K)
    # FP8 cast: bf16 in, E4M3 codes + one fp32 scale per 128 channels out
    assert bench.bytes_pack(N, H, K, R, ROWS, kind="cast", meta=False) == N * 2 * H + N * R * 4 + \
        ROWS * (H + 4 * (H // 128))
    # pre-quantised FP8 in: codes and scales read, the same out
    assert bench.bytes_pack(N, H, K, R, ROWS, kind="fp8", meta=False) == N * H + N * R * 4 + \
        ROWS * (H + 4 * (H // 128)) + N * 4 * (H // 128)


def test_layout_and_notify_bytes():
    # layout: top-k read (8K per token), membership written (R), counts out
    assert bench.bytes_layout(N, K, R, E, S) == N * K * 8 + N * R + S * (R + E) * 4
    # 64 ranks add the RDMA-group counts (8 groups)
    assert bench.bytes_layout(16384, K, 64, E, 64) == 16384 * K * 8 + 16384 * 64 + 64 * (64 + E + 8) * 4
    # notify: membership read, send_head written, counts in, the two channel
    # prefix matrices and the rank prefix out, offsets, expert counts
    assert bench.bytes_notify(N, R, S, C, E) == N * R + N * R * 4 + S * R * 4 + 2 * S * R * C * 4 + \
        (R + 1) * 4 + S * E * 4 + E * 4


def test_relay_combine_bytes():
    # 64 ranks in 8 groups: received rows read (2H) into group partials written
    # and read once (2H bf16 or 4H fp32, plus a 32-byte head row each), the
    # token rows written (2H) after reading one group-row index per group
    Nn, Rr, rows, grows = 16384, 64, 125825, 86699
    base = grows * 32 + rows * 2 * H + Nn * (Rr // 8) * 4 + Nn * 2 * H
    w = rows * 4 * K + 2 * grows * 4 * K + Nn * 4 * K
    assert bench.bytes_relay_combine(Nn, H, K, Rr, rows, grows) == base + 2 * grows * 2 * H + w
    assert bench.bytes_relay_combine(Nn, H, K, Rr, rows, grows, partial_f32=True) == base + 2 * grows * 4 * H + w


def test_ll_bytes():
    # FP8 message: 16-byte header + H codes + H/128 fp32 scales = 7408 bytes
    msgs, toks, Hh, L, Rr = 1024, 930, 7168, 8, 32
    mb = 16 + Hh + 4 * (Hh // 128)
    assert mb == 7408
    assert bench.bytes_ll(msgs, toks, Hh, True, Rr, L) == toks * 2 * Hh + msgs * mb + msgs * (mb - 16 + 4) + \
        L * Rr * 12


def test_rows_match_an_independent_count():
    # the receive-row count that the formulas take equals the number of
    # (token, rank) pairs of the routing, counted by the brute-force layout
    rng = np.random.default_rng(0)
    Sx, Tx, Ex, Rx, Kx = 3, 11, 12, 4, 3
    idx = np.stack([rng.permutation(Ex)[:Kx] for _ in range(Sx * Tx)]).astype(np.int64)
    idx[rng.random(idx.shape) < 0.2] = -1
    lay = brute.layout(idx, Sx, Ex, Rx)
    rows = sum(map(sum, lay["num_tokens_per_rank"]))
    pairs = sum(len({int(e) // (Ex // Rx) for e in row if e >= 0}) for row in idx)
    assert rows == pairs
    Hx, Nx = 64, Sx * Tx
    assert bench.bytes_combine(Nx, Hx, Kx, Rx, rows) == rows * 2 * Hx + Nx * Rx * 4 + Nx * 2 * Hx + \
        rows * 4 * Kx + Nx * 4 * Kx


def test_normal_receive_rows():
    # the seed-0 normal routing sends 21626 (token, rank) rows (5.28 per token)
    import oracle
    from combine_get_dispatch_histogram_amd import workloads as wl
    idx = wl.normal_inputs(wl.NORMAL, 0)["topk_idx"].numpy()
    lay = oracle.layout(idx, S, E, R)
    assert int(lay["num_tokens_per_rank"].sum()) == ROWS
