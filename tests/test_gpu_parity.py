"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small sizes are compared in full (several tiles and a ragged tail); the five
measured workloads run at full size in the benchmark's launch configuration
and are compared on sampled rows.
"""
import numpy as np
import pytest

from tests.parity import check_attention, check_selection, bf16_to_f64

pytestmark = pytest.mark.gpu


def log(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_csa2_amd as csa2
    csa2.lib()
    return "cuda"


def _up(a):
    import csa2_harness
    return csa2_harness.up(a)


def _down(t):
    import csa2_harness
    return csa2_harness.down(t)


# ---------------------------------------------------------------- formats
def test_fp4_decode_matches_oracle_values(dev, orc):
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    log("csa2_decode_fp4_rows: 256 code bytes x scale bytes")
    sbytes = np.array([1, 60, 100, 117, 120, 125, 127, 128, 130, 140, 180, 250], np.uint8)
    rows = len(sbytes)
    codes = np.tile(np.arange(256, dtype=np.uint8)[None, :16 * 16], (rows, 1))  # 256 bytes = 512 elems
    scales = np.repeat(sbytes[:, None], 16, axis=1)
    out = torch.zeros(rows, 512, dtype=torch.bfloat16, device=dev)
    csa2.csa2_decode_fp4_rows(_up(codes), _up(scales), out)
    torch.cuda.synchronize()
    got = bf16_to_f64(_down(out))
    ref = orc.fp4_decode(codes, scales)
    assert np.array_equal(got, ref)


def test_fp8_decode_matches_oracle_values(dev, orc):
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    log("csa2_decode_fp8_rows: all 254 finite codes")
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0, 0x80        # NaN codes are never stored
    out = torch.zeros(1, 256, dtype=torch.bfloat16, device=dev)
    csa2.csa2_decode_fp8_rows(_up(codes[None]), out)
    torch.cuda.synchronize()
    got = bf16_to_f64(_down(out))[0]
    ref = np.array([orc.e4m3_value(int(c)) for c in codes])
    assert np.array_equal(got, ref)


def _edge_rows(rng, cols):
    x = rng.standard_normal((64, cols)).astype(np.float32)
    x[1] *= 1e-3
    x[2] *= 300.0
    x[3] = 0.0
    x[4, ::7] = 0.0
    x[5] = np.ldexp(np.round(rng.standard_normal(cols) * 4) / 4, rng.integers(-3, 3, cols))  # ties
    x[6] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], cols) * rng.choice([-1, 1], cols)
    x[7] = np.exp(rng.standard_normal(cols) * 3) * rng.choice([-1, 1], cols)
    import tests.test_oracle_compress as tc
    return tc.bf16(x)


def test_encoders_bit_exact(dev, orc):
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    rng = np.random.default_rng(5)
    for cols in (512, 128):
        x = _edge_rows(rng, cols)
        log(f"csa2_encode_fp4_rows / fp8_rows: rows={len(x)} cols={cols}")
        c4 = torch.zeros(len(x), cols // 2, dtype=torch.uint8, device=dev)
        s4 = torch.zeros(len(x), cols // 32, dtype=torch.uint8, device=dev)
        c8 = torch.zeros(len(x), cols, dtype=torch.uint8, device=dev)
        s8 = torch.zeros(len(x), dtype=torch.float32, device=dev)
        xd = _up(x)
        csa2.csa2_encode_fp4_rows(xd, c4, s4)
        csa2.csa2_encode_fp8_rows(xd, c8, s8)
        torch.cuda.synchronize()
        oc4, os4 = orc.fp4_encode_rows_bf16(x)
        oc8, os8 = orc.fp8_encode_rows_bf16(x)
        assert np.array_equal(_down(c4), oc4) and np.array_equal(_down(s4), os4)
        assert np.array_equal(_down(c8), oc8) and np.array_equal(_down(s8), os8)
        # the pages' per-16 E4M3 format, and its dequantisation
        ce = torch.zeros(len(x), cols // 2, dtype=torch.uint8, device=dev)
        se = torch.zeros(len(x), cols // 16, dtype=torch.uint8, device=dev)
        csa2.csa2_encode_fp4e4_rows(xd, ce, se)
        de = torch.zeros(len(x), cols, dtype=torch.bfloat16, device=dev)
        csa2.csa2_decode_fp4e4_rows(ce, se, de)
        torch.cuda.synchronize()
        oce, ose = orc.fp4e4_encode_rows_bf16(x)
        assert np.array_equal(_down(ce), oce) and np.array_equal(_down(se), ose)
        assert np.array_equal(bf16_to_f64(_down(de)), orc.fp4e4_decode(oce, ose))


# ---------------------------------------------------------------- prefill
def _prefill(wl):
    import torch
    import csa2_harness
    log(f"csa2_forward prefill: {wl.name} seed={wl.seed:#x}")
    run = csa2_harness.PrefillRun(wl)
    run.forward()
    torch.cuda.synchronize()
    return run


def _check_prefill_rows(wl, out, ref, rows, attn=True):
    r = ref.rows(rows, want_scores=True, want_attn=attn)
    swaps = 0
    for i, t in enumerate(rows):
        swaps += check_selection(out["idx"][0, t], out["cnt"][0, t], r["idx"][i], r["cnt"][i],
                                 r["S"][i])
    if attn:
        import oracle
        got = out["O"][0][:, rows, :].transpose(1, 0, 2)
        exp = r["O"]
        # where a boundary swap changed the row set, evaluate the oracle on the GPU's selection
        for i, t in enumerate(rows):
            if not np.array_equal(out["idx"][0, t], r["idx"][i]):
                O, _, _ = oracle.attend(wl.Q_rows(0, [t])[0], int(t), ref.w_codes[0],
                                        ref.w_scale[0], ref.cap, ref.z_codes[0], ref.z_scales[0],
                                        out["idx"][0, t], int(out["cnt"][0, t]), ref.sink,
                                        ref.cos, ref.sin, z_format=wl.z_format)
                exp = exp.copy()
                exp[i] = O
        mx, rel = check_attention(got, exp, wl.name)
        log(f"  rows={len(rows)} swaps={swaps} max|dO|={mx:.2e} rel={rel:.2e}")
    return swaps


@pytest.mark.parametrize("T,H", [(256, 16), (257, 16), (130, 32)])
def test_prefill_derived_keys_full(dev, synth, T, H):
    """T=256 is the small measured workload; odd T leaves the last position pending."""
    from oracle.reference import PrefillReference
    wl = synth.workload(0, T=T, H=H)
    out = _prefill(wl).fetch()
    ref = PrefillReference(wl)
    w_codes, w_scale = ref.window_full()
    n = T // 2
    assert np.array_equal(out["z_codes"][0, :n], ref.z_codes[0, :n])
    assert np.array_equal(out["z_scales"][0, :n], ref.z_scales[0, :n])
    assert np.array_equal(out["ki_codes"][0, :n], ref.ki_codes[0, :n])
    assert np.array_equal(out["ki_scales"][0, :n], ref.ki_scales[0, :n])
    assert np.array_equal(out["w_codes"][0, :T], w_codes[:T])
    assert np.array_equal(out["w_scale"][0, :T], w_scale[:T])
    _check_prefill_rows(wl, out, ref, np.arange(T))


def test_prefill_clustered_keys_ragged(dev, synth):
    """given-mode keys, 2 index chunks + a ragged tail, selection active for t >= 1023"""
    from oracle.reference import PrefillReference
    wl = synth.workload(1, T=2600, H=16)
    out = _prefill(wl).fetch()
    ref = PrefillReference(wl)
    n = wl.Tq // 2
    assert np.array_equal(out["z_codes"][0, :n], ref.z_codes[0, :n])
    assert np.array_equal(out["ki_codes"][0, :n], ref.ki_codes[0, :n])
    assert np.array_equal(out["ki_scales"][0, :n], ref.ki_scales[0, :n])
    rows = np.unique(np.concatenate([np.arange(0, 8), [1021, 1022, 1023, 1024, 2047, 2048],
                                     np.arange(wl.Tq - 6, wl.Tq),
                                     np.random.default_rng(3).integers(0, wl.Tq, 30)]))
    _check_prefill_rows(wl, out, ref, rows)


@pytest.mark.parametrize("cid,T,H,zf", [(0, 257, 16, 0), (1, 1400, 16, 0), (0, 257, 16, 1),
                                         (1, 1400, 32, 1)])
def test_prefill_ratio_one(dev, synth, cid, T, H, zf):
    """compression ratio one: T entries, entry t rotated at t, a query at t sees entries
    0..t (top-512 active from t = 512 on); caches bit-exact, rows against the oracle.
    zf = 1: compressed rows in the pages' per-16 E4M3 format (dequantising attention)"""
    from oracle.reference import PrefillReference
    wl = synth.workload(cid, T=T, H=H, ratio=1, z_format=zf)
    out = _prefill(wl).fetch()
    ref = PrefillReference(wl)
    for k in ("z_codes", "z_scales", "ki_codes", "ki_scales"):
        assert np.array_equal(out[k][0, :T], getattr(ref, k)[0, :T]), k
    rows = np.arange(T) if T < 300 else np.unique(np.concatenate(
        [np.arange(0, 6), [510, 511, 512, 513, 1023], np.arange(T - 5, T),
         np.random.default_rng(5).integers(0, T, 30)]))
    assert np.all(out["cnt"][0, rows] == np.minimum(rows + 1, 512))
    _check_prefill_rows(wl, out, ref, rows)


@pytest.mark.parametrize("T,H", [(256, 16), (131, 48)])
def test_prefill_pages_z_format(dev, synth, T, H):
    """ratio 2 with compressed rows in the pages' per-16 E4M3 format: caches bit-exact
    (288-byte entries), every row's selection and attention against the oracle"""
    from oracle.reference import PrefillReference
    wl = synth.workload(0, T=T, H=H, z_format=1)
    out = _prefill(wl).fetch()
    ref = PrefillReference(wl)
    n = T // 2
    assert out["z_scales"].shape[2] == 32
    for k in ("z_codes", "z_scales", "ki_codes", "ki_scales"):
        assert np.array_equal(out[k][0, :n], getattr(ref, k)[0, :n]), k
    _check_prefill_rows(wl, out, ref, np.arange(T))


def test_prefill_deterministic(dev, synth):
    import torch
    import csa2_harness
    wl = synth.workload(1, T=1500, H=32)
    log(f"determinism: {wl.name}")
    run = csa2_harness.PrefillRun(wl)
    run.forward()
    a = run.fetch()
    run.idx.fill_(-5)
    run.O.zero_()
    run.forward()
    torch.cuda.synchronize()
    b = run.fetch()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_sparse_attn_given_oracle_selection(dev, synth):
    """attention alone, fed the oracle's caches and selections"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    from oracle.reference import PrefillReference
    wl = synth.workload(1, T=1400, H=64)
    ref = PrefillReference(wl)
    w_codes, w_scale = ref.window_full()
    rows = np.arange(wl.Tq)
    sel = ref.rows(rows, want_attn=False)
    log(f"csa2_sparse_attn with oracle selection: {wl.name}")
    O = torch.zeros(1, wl.H, wl.Tq, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(1, wl.H, wl.Tq, dtype=torch.float32, device=dev)
    cos_t, sin_t = synth.rope_table(wl.rope_rows)
    ws = csa2.workspace(csa2.OP_SPARSE_ATTN, 1, wl.Tq, wl.H, wl.Tq // 2)
    csa2.csa2_sparse_attn(_up(np.zeros(1, np.int32)), _up(wl.Q()), _up(w_codes[None]),
                          _up(w_scale[None]), _up(ref.z_codes), _up(ref.z_scales),
                          _up(sel["idx"][None]), _up(sel["cnt"][None]), _up(ref.sink),
                          _up(cos_t), _up(sin_t), O, lse, ws)
    torch.cuda.synchronize()
    sample = np.random.default_rng(9).choice(wl.Tq, 40, replace=False)
    r = ref.rows(sample)
    got = _down(O)[0][:, sample, :].transpose(1, 0, 2)
    mx, rel = check_attention(got, r["O"], "sparse_attn")
    lse_g = _down(lse)[0][:, sample].T
    assert np.max(np.abs(lse_g - r["lse"])) < 1e-3
    log(f"  max|dO|={mx:.2e} rel={rel:.2e}")


@pytest.mark.parametrize("zf,Tq,H", [(0, 5, 64), (1, 5, 64), (0, 30, 64), (0, 30, 32)])
def test_sparse_attn_bounded_replay_floor(dev, synth, zf, Tq, H):
    """attention with a per-request replay start s: request 0 none, request 1 a start
    inside the 128-row window, request 2 a start past every query (one window row);
    zf = 1: compressed rows in the pages' per-16 E4M3 format.  Tq=30: 90 query rows,
    which the attention kernel runs as two head groups a row (32 or 16 heads each)"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import oracle
    from oracle.reference import DecodeReference
    B, N = 3, 2600
    wl = synth.decode_workload(B=B, Tq=Tq, n_entries=N, H=H, z_format=zf)
    p0 = wl.q_pos0
    floors = np.array([0, p0 - 40, p0 + 100], np.int32)
    log(f"csa2_sparse_attn with replay starts {floors.tolist()}: {wl.name}")
    g = np.random.default_rng(17)
    cnts = np.array([[512, 300, 1, 0, 512] * (Tq // 5)] * B, np.int32)
    idx = np.full((B, Tq, 512), -1, np.int32)
    refs = [DecodeReference(wl, b) for b in range(B)]
    for b in range(B):
        for i in range(Tq):
            c = cnts[b, i]
            idx[b, i, :c] = np.sort(g.choice(N, c, replace=False))
        refs[b]._ensure_z(idx[b].reshape(-1))
    O = torch.zeros(B, H, Tq, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, Tq, dtype=torch.float32, device=dev)
    cos_t, sin_t = synth.rope_table(wl.rope_rows)
    ws = csa2.workspace(csa2.OP_SPARSE_ATTN, B, Tq, H, N)
    stack = lambda name: _up(np.stack([getattr(r, name) for r in refs]))
    csa2.csa2_sparse_attn(_up(np.full(B, p0, np.int32)), _up(wl.Q()), stack("w_codes"),
                          stack("w_scale"), stack("z_codes"), stack("z_scales"), _up(idx),
                          _up(cnts), _up(refs[0].sink), _up(cos_t), _up(sin_t), O, lse, ws,
                          win_floor=_up(floors), z_format=zf)
    torch.cuda.synchronize()
    got_O, got_lse = _down(O), _down(lse)
    Q = wl.Q()
    for b in range(B):
        r = refs[b]
        exp = np.zeros((Tq, H, 512))
        exp_lse = np.zeros((Tq, H))
        for i in range(Tq):
            exp[i], exp_lse[i], _ = oracle.attend(Q[b][:, i, :], p0 + i, r.w_codes, r.w_scale,
                                                  wl.cap, r.z_codes, r.z_scales, idx[b, i],
                                                  int(cnts[b, i]), r.sink, r.cos, r.sin,
                                                  w_floor=int(floors[b]), z_format=zf)
        mx, rel = check_attention(got_O[b].transpose(1, 0, 2), exp, f"floor {floors[b]}")
        assert np.max(np.abs(got_lse[b].T - exp_lse)) < 1e-3
        log(f"  request {b} (s={floors[b]}): max|dO|={mx:.2e} rel={rel:.2e}")


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("Tq,N,keys,ratio,zf", [(1, 3000, "flat", 2, 0),
                                                (6, 2600, "lognormal_dup", 2, 0),
                                                (6, 2600, "lognormal_dup", 1, 0),
                                                (1, 700, "flat", 1, 0),
                                                (6, 2600, "lognormal_dup", 1, 1),
                                                (1, 3000, "flat", 2, 1)])
def test_decode_small(dev, synth, Tq, N, keys, ratio, zf):
    """ratio 1: one entry per position, a query at p sees entries 0..p (700 entries: every
    one selectable only up to 512, the window and the entries overlap); zf = 1: the
    pages' per-16 E4M3 compressed rows"""
    import torch
    import csa2_harness
    from oracle.reference import DecodeReference
    wl = synth.decode_workload(B=3, Tq=Tq, n_entries=N, H=64, keys=keys, ratio=ratio,
                               z_format=zf)
    log(f"csa2_forward decode: {wl.name} keys={keys}")
    run = csa2_harness.DecodeRun(wl)
    run.forward()
    torch.cuda.synchronize()
    out = run.fetch()
    import oracle
    for b in range(wl.B):
        ref = DecodeReference(wl, b)
        r = ref.rows(np.arange(Tq), want_scores=True)
        swaps = 0
        for i in range(Tq):
            swaps += check_selection(out["idx"][b, i], out["cnt"][b, i], r["idx"][i], r["cnt"][i],
                                     r["S"][i])
        exp = r["O"].copy()
        for i in range(Tq):     # a boundary swap: judge attention on the GPU's selection
            if not np.array_equal(out["idx"][b, i], r["idx"][i]):
                ref._ensure_z(out["idx"][b, i])
                exp[i] = oracle.attend(wl.Q()[b][:, i, :], wl.q_pos0 + i, ref.w_codes, ref.w_scale,
                                       wl.cap, ref.z_codes, ref.z_scales, out["idx"][b, i],
                                       int(out["cnt"][b, i]), ref.sink, ref.cos, ref.sin,
                                       z_format=zf)[0]
        mx, rel = check_attention(out["O"][b].transpose(1, 0, 2), exp, wl.name)
        log(f"  request {b}: swaps={swaps} max|dO|={mx:.2e} rel={rel:.2e}")


def test_index_scores_match_oracle(dev, orc):
    """raw indexer scores against the oracle's (fp32 accumulation vs exact), ragged chunks"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(17)
    N, Tq = 2100, 12
    kpre = tc.bf16(rng.standard_normal((N, 128)).astype(np.float32))
    kc_, ks_ = orc.fp4_encode_rows_bf16(kpre)
    qI = tc.bf16(rng.standard_normal((1, Tq, 32, 128)).astype(np.float32))
    wI = (rng.standard_normal((1, Tq, 32)) / 64).astype(np.float32)
    q0 = 2 * N - Tq - 300            # last queries see every entry
    log(f"csa2_index_scores: N={N} Tq={Tq}")
    S = torch.full((1, Tq, N), float("nan"), dtype=torch.float32, device=dev)
    ws = csa2.workspace(csa2.OP_INDEX_SCORES, 1, Tq, 64, N)
    csa2.csa2_index_scores(_up(np.array([q0], np.int32)), _up(np.array([N], np.int32)), _up(qI),
                           _up(wI), _up(kc_[None]), _up(ks_[None]), S, ws)
    torch.cuda.synchronize()
    g = _down(S)[0]
    e4 = np.array([orc.e4m3_value(c) for c in range(256)])
    Kabs = np.abs(orc.fp4_decode(kc_, ks_))
    u = 2.0 ** -24
    for i in range(Tq):
        n = min((q0 + i + 1) // 2, N)
        q8, sq = orc.quant_index_query(qI[0, i])
        ref = orc.index_scores(q8, sq, wI[0, i], kc_, ks_, n)
        assert np.all(np.isfinite(g[i, :n]))
        err = np.abs(g[i, :n].astype(np.float64) - ref)
        # fp32 recursive-summation bound: 128-term dot products (<= 127u), the weight
        # product, the 32-term head sum and the final rounding, with a factor-2 margin
        mass = (Kabs[:n] @ (np.abs(e4[q8]).T * (np.abs(wI[0, i]) * sq)[None, :])).sum(1)
        bound = 2 * (128 + 32 + 2) * u * mass + u * np.abs(ref)
        assert np.all(err <= bound), (i, err.max(), (err / bound).max())


@pytest.mark.parametrize("N", [4096, 8192])
def test_topk_sampled_threshold_fallback(dev, orc, N):
    """Lists of 4096 or more scores start from a threshold taken on a sample of
    16 runs of 64 elements (one run every len/16 entries).  Here those runs hold
    every large score, so fewer than 512 scores pass it and the list must be
    streamed again from threshold 0; the selection must still be the exact top
    512 (N=4096: one list; N=8192: two 4096-entry segments and their merge)."""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(23)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    pos = np.arange(N) % 4096
    hot = (pos % 256) < 64
    kpre = 0.3 * rng.standard_normal((N, 128)) + np.where(hot, 3.0, -3.0)[:, None] * u[None, :]
    kc_, ks_ = orc.fp4_encode_rows_bf16(tc.bf16(kpre.astype(np.float32)))
    qI = tc.bf16((4.0 * u[None, None, None, :]
                  + 0.3 * rng.standard_normal((1, 1, 32, 128))).astype(np.float32))
    wI = (np.abs(rng.standard_normal((1, 1, 32))) / 64).astype(np.float32)
    q0 = 2 * N - 1
    q8, sq = orc.quant_index_query(qI[0, 0])
    S = orc.index_scores(q8, sq, wI[0, 0], kc_, ks_, N)
    # the construction does what it is for: in each 4096-entry list the sample's
    # 192nd largest score (the rank the kernel aims at) has fewer than 512 above it
    for s0 in range(0, N, 4096):
        seg = S[s0:s0 + 4096]
        smp = np.sort(seg[(np.arange(16)[:, None] * 256 + np.arange(64)[None, :]).ravel()])
        assert np.count_nonzero(seg >= smp[-192]) < 512
    log(f"csa2_index_topk sampled-threshold fallback: N={N}")
    idx = torch.full((1, 1, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1, 1), -7, dtype=torch.int32, device=dev)
    ws = csa2.workspace(csa2.OP_INDEX_TOPK, 1, 1, 64, N)
    csa2.csa2_index_topk(_up(np.array([q0], np.int32)), _up(np.array([N], np.int32)), _up(qI),
                         _up(wI), _up(kc_[None]), _up(ks_[None]), idx, cnt, ws)
    torch.cuda.synchronize()
    r_idx, r_cnt = orc.topk(S, N)
    swaps = check_selection(_down(idx)[0, 0], _down(cnt)[0, 0], r_idx, r_cnt, S)
    assert np.all(hot[r_idx[:r_cnt]])
    log(f"  swaps={swaps}")


# ---------------------------------------------------------------- degenerate calls
def test_degenerate_calls(dev, synth):
    """empty calls write nothing; requests with no compressed entries attend over the window
    alone (cnt 0); a single new token at ratio 2 writes no entry, at ratio 1 one entry"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import oracle
    from oracle.reference import DecodeReference
    B, N, H = 2, 64, 16
    wl = synth.decode_workload(B=B, Tq=3, n_entries=N, H=H)
    log(f"degenerate calls: {wl.name}")
    refs = [DecodeReference(wl, b) for b in range(B)]
    cos_t, sin_t = synth.rope_table(wl.rope_rows)
    g = {k: _up(np.stack([getattr(r, k) for r in refs])) for k in
         ("ki_codes", "ki_scales", "w_codes", "w_scale")}
    for r in refs:
        r._ensure_z(np.arange(N))
    zc, zs = _up(np.stack([r.z_codes for r in refs])), _up(np.stack([r.z_scales for r in refs]))
    q0 = _up(np.full(B, wl.q_pos0, np.int32))
    # Tq = 0: nothing is launched, outputs untouched
    idx0 = torch.full((B, 0, 512), -7, dtype=torch.int32, device=dev)
    ws = csa2.workspace(csa2.OP_INDEX_TOPK, B, 1, H, N)
    csa2.csa2_index_topk(q0, _up(np.full(B, N, np.int32)), _up(wl.qI()[:, :0]),
                         _up(wl.wI()[:, :0]), g["ki_codes"], g["ki_scales"], idx0,
                         torch.zeros(B, 0, dtype=torch.int32, device=dev), ws)
    # n_entries = 0 for request 0, 5 for request 1: counts 0 and 5
    ne = np.array([0, 5], np.int32)
    idx = torch.full((B, 3, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, 3), -7, dtype=torch.int32, device=dev)
    csa2.csa2_index_topk(q0, _up(ne), _up(wl.qI()), _up(wl.wI()), g["ki_codes"], g["ki_scales"],
                         idx, cnt, csa2.workspace(csa2.OP_INDEX_TOPK, B, 3, H, N))
    torch.cuda.synchronize()
    c, ix = _down(cnt), _down(idx)
    assert np.all(c[0] == 0) and np.all(ix[0] == -1)
    assert np.all(c[1] == 5) and np.all(ix[1][:, :5] == np.arange(5)) and np.all(ix[1][:, 5:] == -1)
    for zf in (0, 1):
        if zf == 1:
            zs1 = [oracle.fp4e4_encode_rows_bf16(synth.normal(wl.seed, 14, (N, 512)))
                   for _ in range(B)]
            zc_, zs_ = _up(np.stack([a for a, _ in zs1])), _up(np.stack([b_ for _, b_ in zs1]))
            zc_h, zs_h = [a for a, _ in zs1], [b_ for _, b_ in zs1]
        else:
            zc_, zs_ = zc, zs
            zc_h, zs_h = [r.z_codes for r in refs], [r.z_scales for r in refs]
        O = torch.zeros(B, H, 3, 512, dtype=torch.bfloat16, device=dev)
        lse = torch.zeros(B, H, 3, dtype=torch.float32, device=dev)
        csa2.csa2_sparse_attn(q0, _up(wl.Q()), g["w_codes"], g["w_scale"], zc_, zs_, idx, cnt,
                              _up(refs[0].sink), _up(cos_t), _up(sin_t), O, lse,
                              csa2.workspace(csa2.OP_SPARSE_ATTN, B, 3, H, N), z_format=zf)
        torch.cuda.synchronize()
        got = _down(O)
        for b in range(B):
            r = refs[b]
            exp = np.stack([oracle.attend(wl.Q()[b][:, i, :], wl.q_pos0 + i, r.w_codes, r.w_scale,
                                          wl.cap, zc_h[b], zs_h[b], ix[b, i], int(c[b, i]), r.sink,
                                          r.cos, r.sin, z_format=zf)[0] for i in range(3)])
            check_attention(got[b].transpose(1, 0, 2), exp, f"degenerate b={b} zf={zf}")
    # one new token: ratio 2 writes no entry (the pair is open), ratio 1 writes entry pos0
    for ratio in (2, 1):
        one = synth.workload(0, T=1, H=16, ratio=ratio)
        zc1 = torch.zeros(1, 4, 256, dtype=torch.uint8, device=dev)
        zs1 = torch.zeros(1, 4, 16, dtype=torch.uint8, device=dev)
        kc1 = torch.zeros(1, 4, 64, dtype=torch.uint8, device=dev)
        ks1 = torch.zeros(1, 4, 4, dtype=torch.uint8, device=dev)
        ct, st = synth.rope_table(4)
        csa2.csa2_compress(_up(np.array([2], np.int32)), _up(one.kc()),
                           _up(one.gc()) if ratio == 2 else None, _up(one.gamma_c()),
                           _up(one.w_ik()), _up(one.gamma_ik()), None, _up(ct), _up(st), zc1, zs1,
                           kc1, ks1, ratio=ratio)
        torch.cuda.synchronize()
        written = np.flatnonzero(_down(zs1)[0].any(axis=1))
        assert list(written) == ([] if ratio == 2 else [2]), (ratio, written)


@pytest.mark.parametrize("Tq", [1, 8, 12])
def test_fused_select_clustered_scores(dev, orc, Tq):
    """the fused scores + selection kernel when scores repeat: every cache row drawn
    from one key (all scores equal: the first 512 entries), from 3 keys (about 2,700
    copies of each score) and from 40 keys (about 200 copies).  The buffer trims then
    cannot always land between 512 and the buffer's keep limit and take the exact
    tie-broken cut instead.  Tq 1, 8 and 12 run the kernel's 1-, 8- and 4-token forms
    (12: a ragged last group); 8,192 entries make two 4,096-entry segments and a merge."""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(97 + Tq)
    B, N = 3, 8192
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    for b, nd in enumerate((1, 3, 40)):
        dc, ds = orc.fp4_encode(rng.standard_normal((nd, 128)).astype(np.float32))
        pick = rng.integers(0, nd, N)
        kc[b], ks[b] = dc[pick], ds[pick]
    qI = tc.bf16(rng.standard_normal((B, Tq, 32, 128)).astype(np.float32))
    wI = (rng.standard_normal((B, Tq, 32)) / 64).astype(np.float32)
    ne = np.full(B, N, np.int32)
    q0 = np.full(B, 2 * N, np.int32)
    log(f"fused selection, repeated scores: B={B} Tq={Tq} N={N}")
    idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, Tq), -7, dtype=torch.int32, device=dev)
    csa2.csa2_index_topk(_up(q0), _up(ne), _up(qI), _up(wI), _up(kc), _up(ks), idx, cnt,
                         csa2.workspace(csa2.OP_INDEX_TOPK, B, Tq, 64, N))
    torch.cuda.synchronize()
    gi, gc_ = _down(idx), _down(cnt)
    for b in range(B):
        for i in range(Tq):
            q8, sq = orc.quant_index_query(qI[b, i])
            S = orc.index_scores(q8, sq, wI[b, i], kc[b], ks[b], N)
            r_idx, r_cnt = orc.topk(S, N)
            if b == 0:
                assert np.array_equal(r_idx, np.arange(512))
            # equal keys give equal scores on both sides: the cut is the same entries
            assert gc_[b, i] == r_cnt and np.array_equal(gi[b, i], r_idx), (b, i)


@pytest.mark.parametrize("N", [1024, 2048, 16384])
def test_fused_select_sampled_start(dev, orc, N):
    """the four-token form of the fused kernel starts lists of 1,024 entries or
    more from a threshold taken on 16 tiles of 16 entries spread evenly over the
    list (over each segment of a list cut into segments), and scans a token again
    from minus infinity when fewer than 512 scores pass it.  The tokens whose query
    follows the keys' common direction (tokens 0 and 1 of each group of four) have
    large scores only in the 16 tiles the whole list's sample reads, and ReLU zeroes
    every other score of theirs.  N <= 4096 (one segment, N=1024 the shortest list
    that takes the sample): fewer than 512 of their scores pass the threshold and
    they take the rescan, then cut a tie of zeros.  N=16384 (four 4,096-entry
    segments, each sampling its own tiles, none of them large): they start from
    a threshold below zero, keep every score and cut a tie of zeros in each segment
    before the merge.  Of the other tokens (random queries) some keep their sampled
    start, some rescan.  All must give the exact top 512."""
    import math
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(29)
    Tq = 12
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    starts = (((2 * np.arange(16) + 1) * N) // 32) & ~15
    hot = np.zeros(N, bool)
    for s0 in starts:
        hot[s0:s0 + 16] = True
    kpre = 0.3 * rng.standard_normal((N, 128)) + np.where(hot, 3.0, -3.0)[:, None] * u[None, :]
    kc_, ks_ = orc.fp4_encode_rows_bf16(tc.bf16(kpre.astype(np.float32)))
    aligned = (np.arange(Tq) % 4) < 2
    qpre = 0.3 * rng.standard_normal((1, Tq, 32, 128))
    qpre[0, aligned] += 4.0 * u
    qpre[0, ~aligned] = rng.standard_normal((int((~aligned).sum()), 32, 128))
    qI = tc.bf16(qpre.astype(np.float32))
    wI = (np.abs(rng.standard_normal((1, Tq, 32))) / 64).astype(np.float32)
    q0 = 2 * N
    mean = 256 * 512 / N
    r = math.ceil(mean + 3 * math.sqrt(mean) + 1)
    Ss, above = [], []
    for i in range(Tq):
        q8, sq = orc.quant_index_query(qI[0, i])
        S = orc.index_scores(q8, sq, wI[0, i], kc_, ks_, N)
        Ss.append(S)
        smp = np.sort(np.concatenate([S[s0:s0 + 16] for s0 in starts]))
        above.append(np.count_nonzero(S >= smp[-r]))
    # the construction does what it is for: the aligned tokens' sample has fewer than
    # 512 scores above its r-th largest, or (segments) no segment's sample holds a
    # large score; some random token has more than enough
    if N <= 4096:
        assert all(above[i] < 512 for i in range(Tq) if aligned[i])
        assert any(above[i] >= 512 for i in range(Tq) if not aligned[i])
    else:
        seg_starts = [s0 + ((((2 * q + 1) * 4096) // 32) & ~15)
                      for s0 in range(0, N, 4096) for q in range(16)]
        assert not any(hot[s0:s0 + 16].any() for s0 in seg_starts)
        assert any(above[i] >= 1024 for i in range(Tq) if not aligned[i])
    log(f"fused selection, sampled start and rescan: Tq={Tq} N={N}")
    idx = torch.full((1, Tq, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1, Tq), -7, dtype=torch.int32, device=dev)
    csa2.csa2_index_topk(_up(np.array([q0], np.int32)), _up(np.array([N], np.int32)), _up(qI),
                         _up(wI), _up(kc_[None]), _up(ks_[None]), idx, cnt,
                         csa2.workspace(csa2.OP_INDEX_TOPK, 1, Tq, 64, N))
    torch.cuda.synchronize()
    gi, gc_ = _down(idx), _down(cnt)
    swaps = 0
    for i in range(Tq):
        r_idx, r_cnt = orc.topk(Ss[i], N)
        swaps += check_selection(gi[0, i], gc_[0, i], r_idx, r_cnt, Ss[i])
    log(f"  swaps={swaps}")


@pytest.mark.parametrize("N", [6000, 12000])
def test_single_token_rows_sampled_start(dev, orc, N):
    """single-token rows of 4,096 or more entries on the fused kernel: every segment
    of a row starts from one threshold taken on 16 tiles spread over the row.  Row 0
    puts every large score in those tiles, so too few scores pass and the row is
    scanned again from minus infinity (N=6000: one segment, rescanned in place;
    N=12000: two segments, rescanned by the wave that merges them).  Row 1 has
    random keys (the sampled start holds), row 2 identical keys (every score ties:
    the first 512 entries)."""
    import math
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(31 + N)
    B = 3
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    starts = (((2 * np.arange(16) + 1) * N) // 32) & ~15
    hot = np.zeros(N, bool)
    for s0 in starts:
        hot[s0:s0 + 16] = True
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    kpre = 0.3 * rng.standard_normal((N, 128)) + np.where(hot, 3.0, -3.0)[:, None] * u[None, :]
    kc[0], ks[0] = orc.fp4_encode_rows_bf16(tc.bf16(kpre.astype(np.float32)))
    kc[1], ks[1] = orc.fp4_encode(rng.standard_normal((N, 128)).astype(np.float32))
    one_c, one_s = orc.fp4_encode(rng.standard_normal((1, 128)).astype(np.float32))
    kc[2], ks[2] = one_c[0], one_s[0]
    qpre = rng.standard_normal((B, 1, 32, 128))
    qpre[0, 0] = 4.0 * u + 0.3 * rng.standard_normal((32, 128))
    qI = tc.bf16(qpre.astype(np.float32))
    wI = (np.abs(rng.standard_normal((B, 1, 32))) / 64).astype(np.float32)
    S = []
    for b in range(B):
        q8, sq = orc.quant_index_query(qI[b, 0])
        S.append(orc.index_scores(q8, sq, wI[b, 0], kc[b], ks[b], N))
    # the construction does what it is for: row 0's sample has fewer than 512 scores
    # at or above its r-th largest
    mean = 256 * 512 / N
    r = math.ceil(mean + 4 * math.sqrt(mean) + 2)
    smp = np.sort(np.concatenate([S[0][s0:s0 + 16] for s0 in starts]))
    assert np.count_nonzero(S[0] >= smp[-r]) < 512
    log(f"single-token rows, sampled start: B={B} N={N}")
    idx = torch.full((B, 1, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, 1), -7, dtype=torch.int32, device=dev)
    q0 = np.full(B, 2 * N, np.int32)
    csa2.csa2_index_topk(_up(q0), _up(np.full(B, N, np.int32)), _up(qI), _up(wI), _up(kc), _up(ks),
                         idx, cnt, csa2.workspace(csa2.OP_INDEX_TOPK, B, 1, 64, N))
    torch.cuda.synchronize()
    gi, gc_ = _down(idx), _down(cnt)
    swaps = 0
    for b in range(B):
        r_idx, r_cnt = orc.topk(S[b], N)
        swaps += check_selection(gi[b, 0], gc_[b, 0], r_idx, r_cnt, S[b])
    assert np.array_equal(gi[2, 0], np.arange(512)), "ties: the first 512 entries"
    log(f"  swaps={swaps}")


def test_topk_row_paths(dev, orc):
    """the one-block-per-row selection over score rows (k_topk_row: few rows of more
    than eight tokens a request, 16,384..131,072 cache rows; rows of up to eight
    tokens take the selection without score rows) on its paths: a sampled threshold
    (20,000 candidates), every score kept without a sample (3,000), and the exact
    fallback when the sample cannot separate the scores (all 20,000 keys identical:
    the first 512 entries) or when the large scores sit in one contiguous run
    (entries 5,000..7,499: the wave whose eighth holds them has more candidates than
    room)"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    rng = np.random.default_rng(71)
    B, Tq, N = 4, 9, 20_000
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    for b in range(2):
        kc[b], ks[b] = orc.fp4_encode(rng.standard_normal((N, 128)).astype(np.float32))
    one_c, one_s = orc.fp4_encode(rng.standard_normal((1, 128)).astype(np.float32))
    kc[2], ks[2] = one_c[0], one_s[0]
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    run = (np.arange(N) >= 5000) & (np.arange(N) < 7500)
    kpre = rng.standard_normal((N, 128)) + np.where(run, 3.0, 0.0)[:, None] * u[None, :]
    kc[3], ks[3] = orc.fp4_encode(kpre.astype(np.float32))
    import tests.test_oracle_compress as tc
    qpre = rng.standard_normal((B, Tq, 32, 128))
    qpre[3] = 4.0 * u + 0.3 * rng.standard_normal((Tq, 32, 128))
    qI = tc.bf16(qpre.astype(np.float32))
    wI = (rng.standard_normal((B, Tq, 32)) / 64).astype(np.float32)
    wI[3] = np.abs(wI[3])
    ne = np.array([N, 3000, N, N], np.int32)
    q0 = np.full(B, 2 * N, np.int32)
    log(f"k_topk_row paths: B={B} Tq={Tq} stride={N}")
    idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, Tq), -7, dtype=torch.int32, device=dev)
    csa2.csa2_index_topk(_up(q0), _up(ne), _up(qI), _up(wI), _up(kc), _up(ks), idx, cnt,
                         csa2.workspace(csa2.OP_INDEX_TOPK, B, Tq, 64, N))
    torch.cuda.synchronize()
    gi, gc_ = _down(idx), _down(cnt)
    for b in range(B):
        for i in range(Tq):
            n = int(ne[b])
            q8, sq = orc.quant_index_query(qI[b, i])
            S = orc.index_scores(q8, sq, wI[b, i], kc[b], ks[b], n)
            r_idx, r_cnt = orc.topk(S, n)
            check_selection(gi[b, i], gc_[b, i], r_idx, r_cnt, S)
            if b == 2:
                assert np.array_equal(gi[b, i], np.arange(512)), "ties: the first 512 entries"
            if b == 3:
                # the construction does what it is for: above the sample's threshold
                # (its 105th largest of 1,024 spread scores) one wave's eighth of the
                # row holds more than its 768 slots
                smp = S[(np.arange(1024) * n) >> 10]
                th = np.sort(smp)[::-1][(2048 * 1024 + n - 1) // n - 1]
                per = (n + 2047) // 2048 * 256
                assert max(np.count_nonzero(S[w * per:(w + 1) * per] >= th) for w in range(8)) > 768
