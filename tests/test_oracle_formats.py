"""Pins of the oracle's storage formats and its fp32 exp (no GPU).

FP4 / FP8 are pinned against the OCP bit-field definitions, an independent
brute-force nearest-value search written here in numpy, and (FP8) torch's own
float8_e4m3fn cast; exp against the double-precision libm exp.
"""
import math
import struct

import numpy as np
import pytest
import torch


def f32(x):
    return float(np.float32(x))


# ---------------------------------------------------------------- E2M1
def e2m1_from_bits(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
    return -v if s else v


def test_e2m1_decode_table_matches_bit_fields(orc):
    for code in range(16):
        assert orc.e2m1_value(code) == e2m1_from_bits(code)
    assert sorted({abs(e2m1_from_bits(c)) for c in range(16)}) == [0, .5, 1, 1.5, 2, 3, 4, 6]


def brute_e2m1(y):
    mags = np.array([e2m1_from_bits(c) for c in range(8)])
    a = abs(y)
    if a >= 6:
        c = 7
    else:
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (8 if math.copysign(1.0, y) < 0 else 0)


def test_e2m1_encode_nearest_even_saturating(orc):
    rng = np.random.default_rng(1)
    vals = list(rng.uniform(-9, 9, 4000).astype(np.float32))
    # every midpoint and its fp32 neighbours, both signs, plus zero and saturation
    for mid in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, 100.0]:
        for v in (np.nextafter(np.float32(mid), np.float32(0)), np.float32(mid),
                  np.nextafter(np.float32(mid), np.float32(100))):
            vals += [v, -v]
    vals += [np.float32(0.0), np.float32(-0.0)]
    for v in vals:
        assert orc.e2m1_encode(float(v)) == brute_e2m1(float(v)), v


def test_fp4_block_scale_rule_and_round_trip(orc):
    # exactly representable block round-trips; scale byte = floor(log2 amax) - 2 + 127
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    rng = np.random.default_rng(2)
    for e in (-5, 0, 3):
        x = (rng.choice(mags, 32) * rng.choice([-1, 1], 32)).astype(np.float32) * np.float32(2.0 ** e)
        x[0] = 6.0 * 2.0 ** e       # amax = 1.5 * 2^(e+2)
        codes, scales = orc.fp4_encode(x[None, :])
        assert scales[0, 0] == (e + 2) - 2 + 127
        assert np.array_equal(orc.fp4_decode(codes, scales)[0], x.astype(np.float64))
    # amax a power of two, and one ulp below it
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = 8.0
    assert orc.fp4_encode(x)[1][0, 0] == 3 - 2 + 127
    x[0, 5] = np.nextafter(np.float32(8.0), np.float32(0))
    assert orc.fp4_encode(x)[1][0, 0] == 2 - 2 + 127
    # an all-zero block: scale byte 0, codes 0
    c0, s0 = orc.fp4_encode(np.zeros((1, 32), np.float32))
    assert s0[0, 0] == 0 and not c0.any()
    # values just under 2^(e+3) saturate to 6 * 2^e (code 7)
    x = np.full((1, 32), 7.99, np.float32)
    c7, s7 = orc.fp4_encode(x)
    assert s7[0, 0] == 127 and all(((b & 7) == 7 and (b >> 4) == 7) for b in c7[0])
    # packing: element 2i in the low nibble of byte i
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 6] = 6.0, -0.5, 1.0
    c, s = orc.fp4_encode(x)
    assert c[0, 0] == (7 | (9 << 4)) and c[0, 3] == 2 and s[0, 0] == 127


def test_fp4_error_bound_random(orc):
    # inside the range the error is at most half the local code step; above 6*2^e
    # the value saturates to 6*2^e
    x = np.random.default_rng(3).standard_normal((64, 128)).astype(np.float32)
    c, s = orc.fp4_encode(x)
    d = orc.fp4_decode(c, s)
    for b in range(4):
        blk = slice(32 * b, 32 * b + 32)
        sc = 2.0 ** (s[:, b].astype(np.float64) - 127)[:, None]
        y = np.abs(x[:, blk]) / sc
        half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
        bound = np.where(y > 6, y - 6, half) * sc
        assert np.all(np.abs(d[:, blk] - x[:, blk]) <= bound)


# ---------------------------------------------------------------- E4M3FN
def e4m3_from_bits(code):
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if (code & 0x7F) == 0x7F:
        return float("nan")
    v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


def test_e4m3_decode_table(orc):
    for code in range(256):
        a, b = orc.e4m3_value(code), e4m3_from_bits(code)
        assert (math.isnan(a) and math.isnan(b)) or a == b
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(1) == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
                        np.ldexp(rng.uniform(1, 2, 5000), rng.integers(-12, 9, 5000))]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties -> even)
    vals = np.array([e4m3_from_bits(c) for c in range(0, 126)], np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    v = v[np.abs(v) <= 448.0]      # torch's cast does not saturate (above 448 it gives NaN)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_never_nan(orc):
    for x in (448.0, 449.0, 463.9, 464.0, 1e6, float(np.float32(3e38))):
        assert orc.e4m3_encode(x) == 0x7E and orc.e4m3_encode(-x) == 0xFE


def test_fp8_row_scale(orc):
    x = np.random.default_rng(5).standard_normal(512).astype(np.float32)
    codes, s = orc.fp8_encode_row(x)
    assert s == f32(np.float32(np.abs(x).max()) / np.float32(448.0))
    assert abs(orc.e4m3_value(int(codes[np.abs(x).argmax()]))) == 448.0
    dec = np.array([orc.e4m3_value(int(c)) for c in codes]) * s
    rel = np.abs(dec - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)
    assert rel.max() <= 2.0 ** -4 + 1e-7     # half of E4M3's 3-bit mantissa step
    z, s0 = orc.fp8_encode_row(np.zeros(512, np.float32))
    assert s0 == 1.0 and not z.any()


# ---------------------------------------------------------------- exp
def ulp32(x):
    x = np.float32(x)
    return float(np.nextafter(x, np.float32(np.inf)) - x)


def test_exp_within_two_ulp_of_libm(orc):
    rng = np.random.default_rng(6)
    xs = np.concatenate([-rng.uniform(0, 87, 200000), -rng.uniform(0, 1e-3, 2000),
                         np.arange(-87, 1, 0.5)]).astype(np.float32)
    worst = 0.0
    for x in xs:
        got = orc.exp32(float(x))
        ref = math.exp(float(x))
        worst = max(worst, abs(got - ref) / ulp32(ref))
    assert worst <= 2.0, worst
    assert orc.exp32(0.0) == 1.0
    assert orc.exp32(-87.5) == 0.0 and orc.exp32(-1000.0) == 0.0


# ---------------------------------------------------------------- the pages' Z format
# "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache", section "Deriving the
# 890 bytes per token" (E2M1 values, one one-byte E4M3 scale per 16 channels: 288 bytes
# per 512-wide entry) and "FP4 is a storage choice" (E4M3 block scales as in NVFP4's
# local scaling, no global scale).  Reading: scale = E4M3(max|x| / 6), elements
# E2M1(x / scale), both nearest-even, the elements saturating at 6.
def _e4m3_torch(v):
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_fp4e4_scale_and_codes_against_torch_and_brute_force(orc):
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((40, 512)) * np.exp(rng.standard_normal((40, 1)) * 2)).astype(np.float32)
    x[3, :16] = 0.0                         # a zero block
    x[4, 16:32] = 1e-4                      # max/6 below half the smallest E4M3 step: scale 0
    codes, scales = orc.fp4e4_encode(x)
    assert codes.shape == (40, 256) and scales.shape == (40, 32)
    for r in range(40):
        for g in range(32):
            blk = x[r, 16 * g:16 * g + 16]
            amax = np.float32(np.max(np.abs(blk)))
            sc = _e4m3_torch(np.float32(amax / np.float32(6.0)))
            assert scales[r, g] == sc, (r, g)
            s = np.float32(e4m3_from_bits(sc))
            for i in range(16):
                k = 16 * g + i
                c = (codes[r, k // 2] >> (4 * (k & 1))) & 15
                want = 0 if s == 0 else brute_e2m1(float(np.float32(blk[i]) / s))
                assert c == want, (r, k)
    assert not codes[3, :8].any() and scales[3, 0] == 0
    assert scales[4, 1] == 0 and not codes[4, 8:16].any()


def test_fp4e4_decode_and_round_trip(orc):
    rng = np.random.default_rng(32)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    svals = np.array([e4m3_from_bits(c) for c in range(1, 127)], np.float64)
    x = np.zeros((8, 512), np.float32)
    for r in range(8):
        for g in range(32):
            s = rng.choice(svals[20:110])
            v = rng.choice(mags, 16) * rng.choice([-1, 1], 16)
            v[rng.integers(16)] = 6.0 * rng.choice([-1, 1])      # amax = 6 s exactly
            x[r, 16 * g:16 * g + 16] = (v * s).astype(np.float32)
    codes, scales = orc.fp4e4_encode(x)
    dec = orc.fp4e4_decode(codes, scales)
    assert np.array_equal(dec, x.astype(np.float64))
    # decode is code value times scale value, from the bit fields
    k = np.arange(512)
    for r in range(2):
        c = (codes[r, k // 2] >> (4 * (k & 1))) & 15
        ref = np.array([e2m1_from_bits(int(a)) * e4m3_from_bits(int(scales[r, i // 16]))
                        for i, a in enumerate(c)])
        assert np.array_equal(dec[r], ref)


def test_fp4e4_error_bound_random(orc):
    """|x - dec| <= s: half the widest E2M1 gap (2) below saturation, and at most
    6 s (1/(1 - 2^-4) - 1) < s above it (s = amax/6 rounded to 4 significant bits)"""
    rng = np.random.default_rng(33)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    codes, scales = orc.fp4e4_encode(x)
    dec = orc.fp4e4_decode(codes, scales)
    s = np.array([[e4m3_from_bits(int(b)) for b in row] for row in scales]).repeat(16, axis=1)
    assert np.all(np.abs(dec - x) <= s + 0.0)
    # finer than the per-32 power-of-two format on the same data, on average
    c0, s0 = orc.fp4_encode(x)
    d0 = orc.fp4_decode(c0, s0)
    assert np.mean((dec - x) ** 2) < np.mean((d0 - x) ** 2)
