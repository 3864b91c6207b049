"""Pins of the oracle's indexer, top-k and sparse attention (no GPU).

Indexer: S(q) - S(-q) removes the ReLU and must equal the plain weighted dot
product (numpy matmul); zero weights give zero scores and the tie rule's
selection.  Top-k: brute force on small inputs with forced ties.  Attention:
the sink identity against torch's float64 SDPA, the t=0 closed form, MQA
symmetry, the 640-row budget and the inverse rotation undoing the window
rotation.
"""
import math

import numpy as np
import pytest
import torch

D = 512
rng = np.random.default_rng(21)


def bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_table(orc):
    return np.array([orc.e4m3_value(c) for c in range(256)], np.float64)


def rand_keys(orc, n):
    x = rng.standard_normal((n, 128)).astype(np.float32)
    return orc.fp4_encode(x)


# ---------------------------------------------------------------- indexer
def test_relu_difference_is_linear_form(orc):
    n = 300
    kc, ks = rand_keys(orc, n)
    K = orc.fp4_decode(kc, ks)                                  # [n, 128] exact
    q = bf16(rng.standard_normal((32, 128)).astype(np.float32))
    w = (rng.standard_normal(32) / 64).astype(np.float32)
    q8, sq = orc.quant_index_query(q)
    qn8, sqn = orc.quant_index_query(q ^ np.uint16(0x8000))    # -q
    assert np.array_equal(sq, sqn) and np.array_equal(qn8, q8 ^ np.uint8(0x80))
    Sp = orc.index_scores(q8, sq, w, kc, ks, n).astype(np.float64)
    Sm = orc.index_scores(qn8, sqn, w, kc, ks, n).astype(np.float64)
    Qd = e4m3_table(orc)[q8] * sq[:, None].astype(np.float64)  # dequantised queries [32,128]
    lin = (w.astype(np.float64)[None, :] * (K @ Qd.T)).sum(1)   # sum_h w_h (q_h . k_j)
    scale = np.abs(Sp).max() + np.abs(Sm).max()
    assert np.max(np.abs((Sp - Sm) - lin)) < 4e-7 * scale
    # with every weight positive and every dot product positive, S is the linear form
    wpos = np.abs(w)
    Sabs = orc.index_scores(q8, sq, wpos, kc, ks, n).astype(np.float64)
    dots = K @ Qd.T
    assert np.all(Sabs >= 0)
    full = np.all(dots > 0, axis=1)
    lin_pos = (wpos.astype(np.float64)[None, :] * np.maximum(dots, 0)).sum(1)
    assert np.allclose(Sabs, lin_pos, rtol=1e-6, atol=0)
    assert np.any(~full)


def test_index_scores_direct_definition_signed_weights(orc):
    """The indexer equation of "DeepSeek V4.1 -- Pooled group -> Source layer, pairs
    pooled" evaluated directly in float64 numpy: S[j] = sum_h w_h * max(q_h . k_j, 0)
    with weights of both signs and dot products of both signs, on the exact decoded
    values of the FP8 queries and FP4 keys.  The placements of the ReLU and of the
    weight that a kernel could plausibly get wrong -- max(w_h d_h, 0), |w_h| max(d_h, 0),
    or no ReLU -- each differ from it by far more than the fp32 rounding allowed here."""
    n = 600
    kc, ks = rand_keys(orc, n)
    K = orc.fp4_decode(kc, ks)                                   # [n, 128] exact values
    q = bf16(rng.standard_normal((32, 128)).astype(np.float32))
    w = (rng.standard_normal(32) / 64).astype(np.float32)
    w[:16] = np.abs(w[:16])                                      # both signs present
    w[16:] = -np.abs(w[16:])
    q8, sq = orc.quant_index_query(q)
    Qd = e4m3_table(orc)[q8] * sq[:, None].astype(np.float64)   # [32, 128] decoded queries
    d = K @ Qd.T                                                 # [n, 32] dot products
    assert (d > 0).mean() > 0.3 and (d < 0).mean() > 0.3
    wd = w.astype(np.float64)[None, :]
    direct = (wd * np.maximum(d, 0.0)).sum(1)
    S = orc.index_scores(q8, sq, w, kc, ks, n).astype(np.float64)
    mass = (np.abs(wd) * np.abs(d)).sum(1)
    # the oracle rounds the exact value once to fp32
    assert np.all(np.abs(S - direct) <= 2.0 ** -24 * np.abs(direct) + 1e-12 * mass)
    # each plausible misplacement is caught with a wide margin
    for wrong in (np.maximum(wd * d, 0.0).sum(1), (np.abs(wd) * np.maximum(d, 0.0)).sum(1),
                  (wd * d).sum(1)):
        assert np.max(np.abs(S - wrong) / mass) > 1e-2


def test_zero_weights_zero_scores_and_tie_rule(orc):
    n = 1000
    kc, ks = rand_keys(orc, n)
    q8, sq = orc.quant_index_query(bf16(rng.standard_normal((32, 128)).astype(np.float32)))
    S = orc.index_scores(q8, sq, np.zeros(32, np.float32), kc, ks, n)
    assert not S.any()
    idx, cnt = orc.topk(S, n)
    assert cnt == 512 and np.array_equal(idx, np.arange(512))


def test_weight_scaling_is_exact(orc):
    n = 200
    kc, ks = rand_keys(orc, n)
    q8, sq = orc.quant_index_query(bf16(rng.standard_normal((32, 128)).astype(np.float32)))
    w = (rng.standard_normal(32) / 64).astype(np.float32)
    S1 = orc.index_scores(q8, sq, w, kc, ks, n)
    S2 = orc.index_scores(q8, sq, w * np.float32(4.0), kc, ks, n)
    assert np.array_equal(S2, S1 * np.float32(4.0))


# ---------------------------------------------------------------- top-k
def brute_topk(S, n, k=512):
    if n <= k:
        return np.concatenate([np.arange(n), -np.ones(k - n, int)]), n
    order = np.lexsort((np.arange(n), -S[:n].astype(np.float64)))   # score desc, j asc
    return np.sort(order[:k]), k


@pytest.mark.parametrize("n", [0, 1, 511, 512, 513, 2000, 5000])
def test_topk_brute_force_with_ties(orc, n):
    S = np.round(rng.standard_normal(max(n, 1)) * 4).astype(np.float32)[:n]  # many exact ties
    idx, cnt = orc.topk(S, n)
    ref, rc = brute_topk(S, n)
    assert cnt == rc and np.array_equal(idx, ref)


def test_causal_count_and_640_rows(orc, synth):
    """n(t) = min(512, floor((t+1)/2)); t = 0 has no candidates; 128 + 512 = 640 rows from t = 1023 on"""
    wl = synth.workload(1, T=2048, H=16)
    from oracle.reference import PrefillReference
    ref = PrefillReference(wl)
    t = np.array([0, 1, 2, 3, 1021, 1022, 1023, 2047])
    r = ref.rows(t, want_attn=False)
    assert list(r["cnt"]) == [min(512, (x + 1) // 2) for x in t]
    assert list(r["cnt"] + np.minimum(t + 1, 128)) == [1, 3, 4, 6, 639, 639, 640, 640]
    for i, x in enumerate(t):
        c = r["cnt"][i]
        assert np.all(r["idx"][i, :c] < (x + 1) // 2) and np.all(r["idx"][i, c:] == -1)
        assert np.all(np.diff(r["idx"][i, :c]) > 0)


def test_causal_count_ratio_one(orc, synth):
    """compression ratio one ("Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache",
    CSA2 section): a query at p sees entries j < floor((p+1)/1), i.e. j <= p, its own
    position's entry included; the selection is the brute-force top-512 of those"""
    import oracle
    N = 1500
    kc, ks = rand_keys(orc, N)
    qI = bf16(rng.standard_normal((8, 32, 128)).astype(np.float32))
    wI = (rng.standard_normal((8, 32)) / 64).astype(np.float32)
    pos = np.array([0, 1, 5, 510, 511, 512, 900, 1499])
    r = oracle.query_rows(pos, N, qI, wI, None, kc, ks, None, None, None, None, 128, None,
                          None, None, want_scores=True, ratio=1)
    assert list(r["cnt"]) == [min(512, p + 1) for p in pos]
    for i, p in enumerate(pos):
        ref, rc = brute_topk(r["S"][i], p + 1)
        assert r["cnt"][i] == rc and np.array_equal(r["idx"][i], ref)
    # the same rows at ratio 2 see half as many
    r2 = oracle.query_rows(pos, N, qI, wI, None, kc, ks, None, None, None, None, 128, None,
                           None, None, ratio=2)
    assert list(r2["cnt"]) == [min(512, (p + 1) // 2) for p in pos]


# ---------------------------------------------------------------- attention
def zero_angle_table(rows):
    return np.ones((rows, 32), np.float32), np.zeros((rows, 32), np.float32)


def caches(orc, cap, N, p_last):
    """random FP8 ring holding positions .. p_last, random FP4 entries"""
    wn = bf16(rng.standard_normal((1, cap, D)).astype(np.float32))
    cos_t, sin_t = zero_angle_table(p_last + 1)
    w_codes, w_scale = orc.window_encode(wn, cos_t, sin_t, cap, pos0=p_last - cap + 1)
    zc, zs = orc.fp4_encode(rng.standard_normal((N, D)).astype(np.float32))
    return w_codes[0], w_scale[0], zc, zs, cos_t, sin_t


def rows_of(orc, p, cap, w_codes, w_scale, zc, zs, idx, cnt, floor=0):
    """G = [W[max(0,floor,p-127)..p]; Z[idx]] from the pinned decoders (window rule of the
    pages; floor = the start of a bounded replay)"""
    e4 = e4m3_table(orc)
    pos = np.arange(max(0, floor, p - 127), p + 1)
    Wr = e4[w_codes[pos % cap]] * w_scale[pos % cap][:, None].astype(np.float64)
    Zr = orc.fp4_decode(zc[idx[:cnt]], zs[idx[:cnt]])
    return np.concatenate([Wr, Zr])


def test_sink_identity_against_sdpa(orc):
    cap, N, p, H = 200, 700, 900, 8
    w_codes, w_scale, zc, zs, cos_t, sin_t = caches(orc, cap, N, p)
    idx = np.sort(rng.choice(N, 512, replace=False)).astype(np.int32)
    Q = bf16((rng.standard_normal((H, D)) * 0.3).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    O, lse, Ob = orc.attend(Q, p, w_codes, w_scale, cap, zc, zs, idx, 512, sink, cos_t, sin_t)
    G = torch.from_numpy(rows_of(orc, p, cap, w_codes, w_scale, zc, zs, idx, 512))
    assert G.shape[0] == 640
    q = torch.from_numpy(f32(Q).astype(np.float64))
    Op = torch.nn.functional.scaled_dot_product_attention(q[None], G[None], G[None],
                                                          scale=1 / math.sqrt(D))[0]
    lse_p = torch.logsumexp((q @ G.T) / math.sqrt(D), dim=1)
    s = torch.from_numpy(sink.astype(np.float64))
    expect = torch.sigmoid(lse_p - s)[:, None] * Op
    assert np.max(np.abs(O - expect.numpy())) < 1e-12
    assert np.allclose(lse, torch.logaddexp(lse_p, s).numpy(), rtol=0, atol=1e-12)
    # a sink at -inf reproduces plain softmax attention
    O2, _, _ = orc.attend(Q, p, w_codes, w_scale, cap, zc, zs, idx, 512,
                          np.full(H, -1e30, np.float32), cos_t, sin_t)
    assert np.max(np.abs(O2 - Op.numpy())) < 1e-12
    # weights over rows plus the sink weight sum to one
    A_sink = np.exp(sink.astype(np.float64) - lse)
    A_rows = np.exp(((q @ G.T) / math.sqrt(D)).numpy() - lse[:, None]).sum(1)
    assert np.allclose(A_sink + A_rows, 1.0, atol=1e-12)


def test_pages_z_format_attention_against_sdpa(orc):
    """compressed rows stored in the pages' per-16 E4M3 format are attended as their
    exact decoded values (float64 SDPA over those rows, with the sink)"""
    cap, N, p, H = 200, 600, 900, 4
    w_codes, w_scale, _, _, cos_t, sin_t = caches(orc, cap, 8, p)
    zc, zs = orc.fp4e4_encode((rng.standard_normal((N, D)) * 2).astype(np.float32))
    idx = np.sort(rng.choice(N, 400, replace=False)).astype(np.int32)
    Q = bf16((rng.standard_normal((H, D)) * 0.3).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    O, lse, _ = orc.attend(Q, p, w_codes, w_scale, cap, zc, zs, idx, 400, sink, cos_t, sin_t,
                           z_format=1)
    e4 = e4m3_table(orc)
    pos = np.arange(p - 127, p + 1)
    G = np.concatenate([e4[w_codes[pos % cap]] * w_scale[pos % cap][:, None].astype(np.float64),
                        orc.fp4e4_decode(zc[idx], zs[idx])])
    G = torch.from_numpy(G)
    q = torch.from_numpy(f32(Q).astype(np.float64))
    Op = torch.nn.functional.scaled_dot_product_attention(q[None], G[None], G[None],
                                                          scale=1 / math.sqrt(D))[0]
    lse_p = torch.logsumexp((q @ G.T) / math.sqrt(D), dim=1)
    s = torch.from_numpy(sink.astype(np.float64))
    expect = (torch.sigmoid(lse_p - s)[:, None] * Op).numpy()   # zero angles: R_p = I
    assert np.max(np.abs(O - expect)) < 1e-12
    assert np.allclose(lse, torch.logaddexp(lse_p, s).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("floor", [0, 800, 850, 899, 900])
def test_bounded_replay_window_against_sdpa(orc, floor):
    """Bounded replay from s ("Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV
    Cache", section "Bounded replay trades exact state for cheaper resumption"): the
    query at p sees window positions max(s, p-127)..p; checked against torch's float64
    SDPA over exactly those rows plus the selected ones, with the sink identity."""
    cap, N, p, H = 200, 700, 900, 4
    w_codes, w_scale, zc, zs, cos_t, sin_t = caches(orc, cap, N, p)
    idx = np.sort(rng.choice(N, 300, replace=False)).astype(np.int32)
    Q = bf16((rng.standard_normal((H, D)) * 0.3).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    O, lse, _ = orc.attend(Q, p, w_codes, w_scale, cap, zc, zs, idx, 300, sink, cos_t, sin_t,
                           w_floor=floor)
    G = torch.from_numpy(rows_of(orc, p, cap, w_codes, w_scale, zc, zs, idx, 300, floor))
    assert G.shape[0] == 300 + (p + 1 - max(floor, p - 127))
    q = torch.from_numpy(f32(Q).astype(np.float64))
    Op = torch.nn.functional.scaled_dot_product_attention(q[None], G[None], G[None],
                                                          scale=1 / math.sqrt(D))[0]
    lse_p = torch.logsumexp((q @ G.T) / math.sqrt(D), dim=1)
    sk = torch.from_numpy(sink.astype(np.float64))
    # the inverse rotation of channels 448.. at p is linear: undo it on both sides by
    # comparing before it (p's rotation applied to the SDPA output instead)
    expect = (torch.sigmoid(lse_p - sk)[:, None] * Op).numpy()
    c, s_ = cos_t[p].astype(np.float64), sin_t[p].astype(np.float64)
    e0, e1 = expect[:, 448::2].copy(), expect[:, 449::2].copy()
    expect[:, 448::2] = e0 * c + e1 * s_
    expect[:, 449::2] = -e0 * s_ + e1 * c
    assert np.max(np.abs(O - expect)) < 1e-12
    assert np.allclose(lse, torch.logaddexp(lse_p, sk).numpy(), rtol=0, atol=1e-12)


def test_first_token_closed_form(orc):
    """t = 0: one window row, no compressed entry: O = sigmoid(S_00 - s_h) W_0 (R_0 = I)"""
    cap, H = 128, 4
    wn = bf16(rng.standard_normal((1, 1, D)).astype(np.float32))
    import csa2_synth
    cos_t, sin_t = csa2_synth.rope_table(4)
    w_codes, w_scale = orc.window_encode(wn, cos_t, sin_t, cap, pos0=0)
    zc, zs = np.zeros((1, 256), np.uint8), np.zeros((1, 16), np.uint8)
    Q = bf16(rng.standard_normal((H, D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    O, lse, _ = orc.attend(Q, 0, w_codes[0], w_scale[0], cap, zc, zs, -np.ones(512, np.int32), 0,
                           sink, cos_t, sin_t)
    W0 = e4m3_table(orc)[w_codes[0, 0]] * float(w_scale[0, 0])
    S00 = f32(Q).astype(np.float64) @ W0 / math.sqrt(D)
    sig = 1 / (1 + np.exp(-(S00 - sink)))
    assert np.max(np.abs(O - sig[:, None] * W0[None, :])) < 1e-12


def test_mqa_identical_queries_identical_heads(orc):
    cap, N, p = 130, 600, 700
    w_codes, w_scale, zc, zs, cos_t, sin_t = caches(orc, cap, N, p)
    idx = np.sort(rng.choice(N, 512, replace=False)).astype(np.int32)
    row = bf16(rng.standard_normal(D).astype(np.float32))
    Q = np.stack([row] * 6)
    O, _, _ = orc.attend(Q, p, w_codes, w_scale, cap, zc, zs, idx, 512, np.zeros(6, np.float32),
                         cos_t, sin_t)
    assert all(np.array_equal(O[0], O[h]) for h in range(6))


def test_inverse_rotation_undoes_window_rotation(orc, synth):
    """A query aimed at the window row of its own position p gets ~that row back, un-rotated."""
    p, cap = 777, 128
    cos_t, sin_t = synth.rope_table(p + 1)
    w = rng.standard_normal((1, cap, D)).astype(np.float32)
    wn = bf16(w)
    w_codes, w_scale = orc.window_encode(wn, cos_t, sin_t, cap, pos0=p - cap + 1)
    e4 = e4m3_table(orc)
    Gp = e4[w_codes[0, p % cap]] * float(w_scale[0, p % cap])
    zc, zs = np.zeros((1, 256), np.uint8), np.zeros((1, 16), np.uint8)
    big = bf16((Gp / np.linalg.norm(Gp) * 2000.0).astype(np.float32))[None]
    O, _, _ = orc.attend(big, p, w_codes[0], w_scale[0], cap, zc, zs, -np.ones(512, np.int32), 0,
                         np.array([-1e30], np.float32), cos_t, sin_t)
    x = f32(wn[0, -1]).astype(np.float64)        # the un-rotated window vector at position p
    assert np.max(np.abs(O[0] - x)) < 0.07 * np.max(np.abs(x))
    assert np.max(np.abs(O[0, 448:] - Gp[448:])) > 0.1       # the rotation was really undone
