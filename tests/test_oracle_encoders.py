"""Pins for the oracle's scalar encoders and the per-128 FP8 quantiser.

The E4M3 and bf16 encoders are checked against exact rational nearest-value
search and against torch's library casts; the FP8 scales against numpy's IEEE
fp32 division and exact powers of two.  None of these references shares code
with the oracle.
"""
import math

import numpy as np
import pytest
import torch

import brute


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    for c in range(256):
        v = brute.e4m3_value(c)
        if v is None:
            assert math.isnan(got[c]), c
        else:
            assert got[c] == float(v), (c, got[c], v)
    # the format's landmarks: largest finite 448, smallest subnormal 2^-9, no infinity
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and not np.isinf(got).any()


def _e4m3_tricky_inputs():
    vals = []
    pos = [float(v) for _c, v in brute.E4M3_POS]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)      # exact in fp32: a tie
        vals += [a, b, float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9)))]
    vals += [448.0, 463.99997, 464.0, 464.00003, 479.0, 480.0, 1e6, 3e38, 2.0 ** -10, 2.0 ** -11, 1e-30, 0.0]
    vals += [-v for v in vals]
    rng = np.random.default_rng(0)
    vals += list(rng.standard_normal(400).astype(np.float32) * 50)
    vals += list((rng.random(200) * 2 ** -6).astype(np.float32))
    return np.array(vals, np.float32)


def test_e4m3_encode_matches_exact_search(orc):
    a = _e4m3_tricky_inputs()
    got = orc.e4m3_encode(a)
    want = np.array([brute.e4m3_encode_exact(float(v)) for v in a], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_cast(orc):
    """torch's float32 -> float8_e4m3fn cast is round-to-nearest-even without
    saturation; in [-464, 464] both must agree bit for bit."""
    # every bf16 bit pattern (as fp32) plus 1M random fp32 values
    bf = _f32(np.arange(65536, dtype=np.uint32) << 16)
    rng = np.random.default_rng(1)
    rnd = (rng.standard_normal(1 << 20) * rng.choice([1e-3, 0.1, 1, 30, 300], 1 << 20)).astype(np.float32)
    a = np.concatenate([bf, rnd])
    a = a[np.isfinite(a) & (np.abs(a) <= 464.0)]
    got = orc.e4m3_encode(a)
    want = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_saturates_and_nan(orc):
    a = np.array([464.1, 1e4, np.inf, -np.inf, -1e30, np.nan], np.float32)
    got = orc.e4m3_encode(a).tolist()
    assert got[:5] == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE] and got[5] == 0x7F


def test_bf16_round_matches_torch_cast(orc):
    rng = np.random.default_rng(2)
    a = (rng.standard_normal(1 << 20) * rng.choice([1e-30, 1e-3, 1, 1e3, 1e30], 1 << 20)).astype(np.float32)
    # exact ties: bf16 value + half a bf16 ulp, for even and odd mantissas
    base = (rng.integers(0, 0x7F00, 4096, dtype=np.uint32) << 16)
    ties = _f32(base | 0x8000)
    near = _f32(base | 0x7FFF)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45], np.float32)
    a = np.concatenate([a, ties, -ties, near, special])
    got = orc.bf16_round(a)
    want = brute.bf16_round_lib(a)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]
    nan = orc.bf16_round(np.array([np.nan], np.float32))
    assert np.isnan(orc.bf16_to_f32(nan))[0]


def _rows_for_fp8(seed):
    rng = np.random.default_rng(seed)
    H = 512
    rows = []
    rows.append(rng.standard_normal(H))                      # N(0,1)
    rows.append(rng.standard_normal(H) * 1e-3)               # small: subnormal codes appear
    rows.append(rng.standard_normal(H) * 300)                # large
    r = rng.standard_normal(H)
    r[:128] = 0.0                                            # an all-zero group: amax floor
    r[128:256] *= 1e-7                                       # amax below the floor
    rows.append(r)
    r = rng.standard_normal(H)
    r[256:384] = 448.0 * 2.0 ** rng.integers(-3, 3)          # exact powers of two: ceil-log2 edge
    rows.append(r)
    x = torch.tensor(np.array(rows), dtype=torch.float32).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_quantize_matches_brute(orc, round_scale):
    x = _rows_for_fp8(3)
    codes, sci, ue = orc.fp8_quantize(x, round_scale)
    for i in range(x.shape[0]):
        bc, bs, be = brute.fp8_quantize_row(x[i], round_scale)
        assert codes[i].tolist() == bc, i
        assert np.array_equal(sci[i], np.array(bs, np.float32)), i
        if round_scale:
            assert ue[i].tolist() == [e + 127 for e in be], i


def test_fp8_scale_properties(orc):
    x = _rows_for_fp8(4)
    xf = orc.bf16_to_f32(x).reshape(x.shape)
    G = x.shape[1] // 128
    amax = np.maximum(np.abs(xf).reshape(x.shape[0], G, 128).max(axis=2), np.float32(1e-4)).astype(np.float32)
    # plain scales: correctly rounded fp32 amax / 448 (numpy's IEEE division)
    _c, sci, _u = orc.fp8_quantize(x, False)
    assert np.array_equal(sci, amax / np.float32(448.0))
    # round_scale: exact powers of two with amax * scale in (224, 448]
    codes, sci2, ue = orc.fp8_quantize(x, True)
    m, e = np.frexp(sci2.astype(np.float64))
    assert np.all(m == 0.5)
    ratio = amax.astype(np.float64) / sci2.astype(np.float64)
    assert np.all(ratio <= 448.0) and np.all(ratio > 224.0)
    assert np.array_equal(ue.astype(np.int64) - 127, (e - 1).astype(np.int64))


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_dequant_error_bound(orc, round_scale):
    """Dequantised codes stay within half an E4M3 step: relative 2^-4 in the
    normal range, 2^-10 * scale_inv in the subnormal range."""
    x = _rows_for_fp8(5)
    xf = orc.bf16_to_f32(x).reshape(x.shape).astype(np.float64)
    codes, sci, _u = orc.fp8_quantize(x, round_scale)
    deq = orc.e4m3_decode(codes).reshape(x.shape).astype(np.float64) * np.repeat(sci, 128, axis=1)
    s_inv = np.repeat(sci, 128, axis=1).astype(np.float64)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, s_inv * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - xf) <= bound)
