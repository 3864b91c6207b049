"""Pins of the oracle's compression step (pair gate, RMSNorm, rotation, K^I) and window encode.

No GPU.  Checks use identities the pages or the mathematics fix: gate limits,
softmax from scipy, RMSNorm invariants and the pages' 22.6 value bound,
rotation properties, and the orientation of the index-key projection.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

D = 512


def bf16(x):
    """fp32 -> bf16 bits (nearest even), test-side helper"""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


ID_COS = np.ones(32, np.float32)
ID_SIN = np.zeros(32, np.float32)


def entry(orc, ka, kb, ga, gb, gamma=None, w_ik=None, gamma_ik=None, ki=None, cs=ID_COS, sn=ID_SIN):
    gamma = np.ones(D, np.float32) if gamma is None else gamma
    gamma_ik = np.ones(128, np.float32) if gamma_ik is None else gamma_ik
    if w_ik is None and ki is None:
        ki = np.zeros(128, np.uint16)
    return orc.compress_entry(ka, kb, ga, gb, gamma, w_ik, gamma_ik, ki, cs, sn)


rng = np.random.default_rng(11)


def rand_bf16(n, scale=1.0):
    return bf16(rng.standard_normal(n).astype(np.float32) * scale)


# ---------------------------------------------------------------- pair gate
def test_gate_equal_gates_is_mean(orc):
    ka, kb, g = rand_bf16(D), rand_bf16(D), rand_bf16(D)
    z = entry(orc, ka, kb, g, g)[4]
    kp = (np.float32(0.5) * f32(ka)) + (np.float32(0.5) * f32(kb))   # exact halves, one rounding
    assert np.array_equal(z, orc.rmsnorm(kp, np.ones(D, np.float32)))


def test_gate_large_gap_selects_one_key(orc):
    ka, kb = rand_bf16(D), rand_bf16(D)
    hi, lo = bf16(np.full(D, 60.0)), bf16(np.full(D, -60.0))     # gap 120 > 87 -> weight 0 exactly
    z1 = entry(orc, ka, kb, hi, lo)[4]
    z2 = entry(orc, ka, kb, lo, hi)[4]
    one = np.ones(D, np.float32)
    assert np.array_equal(z1, orc.rmsnorm(f32(ka), one))
    assert np.array_equal(z2, orc.rmsnorm(f32(kb), one))


def test_gate_is_per_channel_softmax(orc):
    ka, kb, ga, gb = rand_bf16(D), rand_bf16(D), rand_bf16(D, 3), rand_bf16(D, 3)
    z = entry(orc, ka, kb, ga, gb)[4]
    w = softmax(np.stack([f32(ga), f32(gb)]).astype(np.float64), axis=0)
    kp = w[0] * f32(ka) + w[1] * f32(kb)
    ref = kp / np.sqrt(np.mean(kp ** 2) + 1e-20)
    assert np.max(np.abs(z - ref)) < 1e-5 * np.max(np.abs(ref))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_invariants(orc):
    for n in (512, 128):
        x = (rng.standard_normal(n) * 3).astype(np.float32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        y = orc.rmsnorm(x, g)
        assert abs(np.sum((y / g).astype(np.float64) ** 2) - n) < 1e-4 * n
        assert np.all(np.abs(y) <= np.abs(g) * math.sqrt(n) * (1 + 1e-6))
        # power-of-two scaling of the input is exact through every step
        assert np.array_equal(orc.rmsnorm(x * np.float32(8.0), g), y)
        # a constant row maps to +-gamma
        c = np.full(n, -2.5, np.float32)
        assert np.allclose(orc.rmsnorm(c, g), -g, rtol=2e-7, atol=0)


def test_value_bound_22_6(orc):
    """P1 '890 bytes': after normalisation and RoPE no number exceeds ~22.6 (= sqrt 512)"""
    ka = np.zeros(D, np.uint16)
    ka[450] = bf16(np.float32(5.0))
    cs, sn = np.full(32, np.cos(0.3), np.float32), np.full(32, np.sin(0.3), np.float32)
    z = entry(orc, ka, ka, ka, ka, cs=cs, sn=sn)[4]
    pair = math.hypot(z[450], z[451])
    assert abs(pair - math.sqrt(512)) < 1e-5 * math.sqrt(512)
    assert math.sqrt(512) == pytest.approx(22.6, abs=0.05)
    for _ in range(20):
        z = entry(orc, rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D), cs=cs, sn=sn)[4]
        assert np.max(np.abs(z)) <= math.sqrt(512) * (1 + 1e-6)


# ---------------------------------------------------------------- rotation
def test_rotation_zero_angle_is_identity_and_preserves_pairs(orc, synth):
    cos_t, sin_t = synth.rope_table(64)
    ka, kb, ga, gb = rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D)
    z0 = entry(orc, ka, kb, ga, gb, cs=cos_t[0], sn=sin_t[0])[4]
    zi = entry(orc, ka, kb, ga, gb)[4]
    assert np.array_equal(z0, zi)                                  # R_0 = I exactly
    z = entry(orc, ka, kb, ga, gb, cs=cos_t[38], sn=sin_t[38])[4]
    assert np.array_equal(z[:448], zi[:448])                       # channels below 448 untouched
    n1 = np.hypot(z[448::2].astype(np.float64), z[449::2])
    n0 = np.hypot(zi[448::2].astype(np.float64), zi[449::2])
    assert np.max(np.abs(n1 - n0) / n0) < 3e-7
    assert not np.allclose(z[448:], zi[448:])


def test_rotation_relative_position(orc, synth):
    """<R_a x, R_b y> = <x, R_(b-a) y>: the rotation depends on position differences only"""
    cos_t, sin_t = synth.rope_table(400)
    x = [rand_bf16(D) for _ in range(4)]
    y = [rand_bf16(D) for _ in range(4)]
    def rot(v, p):
        return entry(orc, *v, cs=cos_t[p], sn=sin_t[p])[4][448:].astype(np.float64)
    for a, b in ((10, 50), (100, 398), (7, 7)):
        lhs = rot(x, a) @ rot(y, b)
        rhs = rot(x, 0) @ rot(y, b - a)
        assert abs(lhs - rhs) < 1e-4


def test_rotation_direction_matches_angle_table(orc, synth):
    """pair (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos): a counter-clockwise turn"""
    ka = np.zeros(D, np.uint16)
    ka[448] = bf16(np.float32(1.0))       # unit vector on the first rotated pair
    cs = np.full(32, 0.0, np.float32)
    sn = np.full(32, 1.0, np.float32)     # quarter turn
    z = entry(orc, ka, ka, ka, ka, cs=cs, sn=sn)[4]
    assert z[448] == 0.0 and z[449] == pytest.approx(math.sqrt(512), rel=1e-6)


# ---------------------------------------------------------------- index keys
def test_index_key_projection_orientation(orc):
    """k^i = c W_IK with W_IK [512 in, 128 out]: W[k][n] = [k == 2n+1] picks c[2n+1]"""
    ka, kb, ga, gb = rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D)
    W = np.zeros((D, 128), np.uint16)
    W[2 * np.arange(128) + 1, np.arange(128)] = bf16(np.float32(1.0))
    g_ik = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    out = entry(orc, ka, kb, ga, gb, w_ik=W, gamma_ik=g_ik)
    c = out[4]                                   # R_0 = I, gamma_C = 1 -> z_pre == c
    assert np.array_equal(out[5], orc.rmsnorm(c[1:256:2].copy(), g_ik))


def test_index_key_rotation_on_64_to_127(orc, synth):
    cos_t, sin_t = synth.rope_table(16)
    ka, kb, ga, gb = rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D)
    W = bf16((rng.standard_normal((D, 128)) / math.sqrt(D)).astype(np.float32))
    a = entry(orc, ka, kb, ga, gb, w_ik=W)[5]
    b = entry(orc, ka, kb, ga, gb, w_ik=W, cs=cos_t[10], sn=sin_t[10])[5]
    assert np.array_equal(a[:64], b[:64]) and not np.allclose(a[64:], b[64:])
    na = np.hypot(a[64::2].astype(np.float64), a[65::2])
    nb = np.hypot(b[64::2].astype(np.float64), b[65::2])
    assert np.max(np.abs(na - nb) / na) < 3e-7


def test_given_mode_encodes_supplied_keys(orc):
    ki = rand_bf16(128)
    out = entry(orc, rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D), ki=ki)
    assert np.array_equal(out[5], f32(ki))
    assert np.array_equal(out[2], orc.fp4_encode(f32(ki)[None])[0][0])


def test_compress_batch_matches_entries_and_positions(orc, synth):
    """entry j pools positions 2j, 2j+1 and is rotated at position 2j"""
    wl = synth.workload(0, T=16)
    cos_t, sin_t = synth.rope_table(16)
    kc, gc = wl.kc(), wl.gc()
    zc, zs, kic, kis = orc.compress(kc, gc, wl.gamma_c(), wl.w_ik(), wl.gamma_ik(), None,
                                    cos_t, sin_t, entry_stride=8)
    for j in range(8):
        e = orc.compress_entry(kc[0, 2 * j], kc[0, 2 * j + 1], gc[0, 2 * j], gc[0, 2 * j + 1],
                               wl.gamma_c(), wl.w_ik(), wl.gamma_ik(), None, cos_t[2 * j],
                               sin_t[2 * j])
        assert np.array_equal(zc[0, j], e[0]) and np.array_equal(zs[0, j], e[1])
        assert np.array_equal(kic[0, j], e[2]) and np.array_equal(kis[0, j], e[3])


# ---------------------------------------------------------------- compression ratio one
# "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache", CSA2 section: ratio one
# is a supported case (the decoder layers use it); entry j is then position j alone.
def test_ratio_one_entry_is_the_equal_gate_pair_of_one_token(orc, synth):
    """the one-position entry equals the pair formula with the token doubled under equal
    gates (weights 1/2 each, exact: k^p = k^c), byte for byte, index key included"""
    cos_t, sin_t = synth.rope_table(64)
    gamma = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    W = bf16((rng.standard_normal((D, 128)) / math.sqrt(D)).astype(np.float32))
    g_ik = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    for _ in range(4):
        ka, g = rand_bf16(D, 3.0), rand_bf16(D)
        one = orc.compress_entry(ka, None, None, None, gamma, W, g_ik, None, cos_t[37], sin_t[37])
        two = orc.compress_entry(ka, ka, g, g, gamma, W, g_ik, None, cos_t[37], sin_t[37])
        for a, b in zip(one, two):
            assert np.array_equal(a, b)


def test_ratio_one_entry_values_in_float64(orc, synth):
    """z = R_p(gamma_C k^c / rms(k^c)) and k^n = R_p(gamma_IK k^i / rms(k^i)), k^i = c W_IK,
    evaluated in float64 from the equations: agree to fp32 rounding"""
    cos_t, sin_t = synth.rope_table(64)
    gamma = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    W = bf16((rng.standard_normal((D, 128)) / math.sqrt(D)).astype(np.float32))
    g_ik = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    ka = rand_bf16(D, 2.0)
    p = 45
    out = orc.compress_entry(ka, None, None, None, gamma, W, g_ik, None, cos_t[p], sin_t[p])
    x = f32(ka).astype(np.float64)
    c = gamma * x / np.sqrt(np.mean(x * x) + 1e-20)
    def rot(v, lo):
        v = v.copy()
        cs, sn = cos_t[p].astype(np.float64), sin_t[p].astype(np.float64)
        a, b = v[lo::2].copy(), v[lo + 1::2].copy()
        v[lo::2], v[lo + 1::2] = a * cs - b * sn, a * sn + b * cs
        return v
    z = rot(c, 448)
    assert np.max(np.abs(out[4] - z)) < 2e-6 * np.max(np.abs(z))
    ki = c @ f32(W).astype(np.float64)
    kn = rot(g_ik * ki / np.sqrt(np.mean(ki * ki) + 1e-20), 64)
    assert np.max(np.abs(out[5] - kn)) < 2e-5 * np.max(np.abs(kn))


@pytest.mark.parametrize("derive", [True, False])
def test_ratio_one_batch_one_entry_per_position(orc, synth, derive):
    """ratio 1 over T positions from an odd start p0: entry p0+i is position i alone,
    rotated at its own position p0+i (not 2j), given keys one per position"""
    wl = synth.workload(0, T=12, ratio=1)
    T, p0 = 12, 21
    cos_t, sin_t = synth.rope_table(2 * (p0 + T) + 1)
    kc = wl.kc()
    ki = None if derive else rand_bf16(T * 128).reshape(1, T, 128)
    w_ik = wl.w_ik() if derive else None
    zc, zs, kic, kis = orc.compress(kc, None, wl.gamma_c(), w_ik, wl.gamma_ik(), ki, cos_t,
                                    sin_t, entry_stride=p0 + T + 3, pos0=p0, ratio=1)
    for i in range(T):
        j = p0 + i
        e = orc.compress_entry(kc[0, i], None, None, None, wl.gamma_c(), w_ik, wl.gamma_ik(),
                               None if derive else ki[0, i], cos_t[j], sin_t[j])
        assert np.array_equal(zc[0, j], e[0]) and np.array_equal(zs[0, j], e[1])
        assert np.array_equal(kic[0, j], e[2]) and np.array_equal(kis[0, j], e[3])
    assert not zc[0, :p0].any() and not zc[0, p0 + T:].any()      # nothing else written
    # the rotation row matters: at 2j the rotated channels would differ
    e2 = orc.compress_entry(kc[0, 0], None, None, None, wl.gamma_c(), w_ik, wl.gamma_ik(),
                            None if derive else ki[0, 0], cos_t[2 * p0], sin_t[2 * p0])
    assert not np.array_equal(zc[0, p0], e2[0])


# ---------------------------------------------------------------- window
def test_window_rows_rotated_at_position_into_ring_slot(orc, synth):
    cap, T = 8, 13
    cos_t, sin_t = synth.rope_table(40)
    wn = rand_bf16(T * D).reshape(1, T, D)
    codes, scale = orc.window_encode(wn, cos_t, sin_t, cap, pos0=20)
    e4 = np.array([orc.e4m3_value(c) for c in range(256)], np.float64)
    for i in range(T - cap, T):            # the last cap positions survive in the ring
        p = 20 + i
        x = f32(wn[0, i]).astype(np.float64)
        c_, s_ = cos_t[p].astype(np.float64), sin_t[p].astype(np.float64)
        r = x.copy()
        r[448::2] = x[448::2] * c_ - x[449::2] * s_
        r[449::2] = x[448::2] * s_ + x[449::2] * c_
        dec = e4[codes[0, p % cap]] * scale[0, p % cap]
        assert np.max(np.abs(dec - r)) <= np.max(np.abs(r)) * 2.0 ** -4


def test_entry_byte_sizes():
    """P4 'Deriving the 890 bytes': index key 128*4/8 + 128/32 = 68 B; with per-32 byte
    scales a 512-wide entry is 256 + 16 = 272 B (the pages' per-16 scale gives 288 B)"""
    assert 128 * 4 // 8 + 128 // 32 == 68
    assert 512 * 4 // 8 + 512 // 32 == 272
    assert 512 * 4 // 8 + 512 // 16 == 288
    assert (3 / 2 + 1) * (288 + 68) == 890


def test_pages_z_format_encodes_the_same_values(orc, synth):
    """z_format 1 stores the same pre-code values in the pages' per-16 E4M3 format;
    the index key keeps its per-32 format"""
    cos_t, sin_t = synth.rope_table(64)
    W = bf16((rng.standard_normal((D, 128)) / math.sqrt(D)).astype(np.float32))
    ka, kb, ga, gb = rand_bf16(D), rand_bf16(D), rand_bf16(D), rand_bf16(D)
    gamma, g_ik = np.ones(D, np.float32), np.ones(128, np.float32)
    a = orc.compress_entry(ka, kb, ga, gb, gamma, W, g_ik, None, cos_t[9], sin_t[9])
    b = orc.compress_entry(ka, kb, ga, gb, gamma, W, g_ik, None, cos_t[9], sin_t[9], z_format=1)
    assert np.array_equal(a[4], b[4]) and np.array_equal(a[5], b[5])
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])
    zc, zs = orc.fp4e4_encode(b[4][None])
    assert np.array_equal(b[0], zc[0]) and np.array_equal(b[1], zs[0]) and len(b[1]) == 32
