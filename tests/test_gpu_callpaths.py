"""GPU parity of the call paths that position arithmetic runs through
("Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache", sections "How to
audit a port or a serving claim" and "Reading the exact layer schedule": a chunk
of a prefill must see the history before it at the right offsets).

* csa2_forward prefill in two chunks over the same caches and window ring,
  against one oracle run over both chunks;
* a batched prefill whose requests start at different positions over caches
  that already hold each request's earlier positions;
* csa2_forward in decode form writing the new tokens' window rows itself;
* a decode at position p over a prefill's caches reproduces prefill row p
  (the same selection, bit for bit; the output within the attention tolerance);
* the index-query E4M3 quantiser, bit-exact against the oracle, at full size.

All at compression ratio 2 and 1.
"""
import dataclasses

import numpy as np
import pytest

from tests.parity import check_attention, check_selection, prefill_rows_parallel

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


class Caches:
    """device caches and window ring for B requests of a prefill workload"""

    def __init__(self, wl, B, stride, cap):
        import torch
        u8 = torch.uint8
        zsb = 32 if wl.z_format == 1 else 16
        self.z_codes = torch.zeros(B, stride, 256, dtype=u8, device="cuda")
        self.z_scales = torch.zeros(B, stride, zsb, dtype=u8, device="cuda")
        self.ki_codes = torch.zeros(B, stride, 64, dtype=u8, device="cuda")
        self.ki_scales = torch.zeros(B, stride, 4, dtype=u8, device="cuda")
        self.w_codes = torch.zeros(B, cap, 512, dtype=u8, device="cuda")
        self.w_scale = torch.zeros(B, cap, dtype=torch.float32, device="cuda")
        self.stride, self.cap = stride, cap


class Inputs:
    """host copies of a prefill workload's tensors (B requests x T_full positions)"""

    def __init__(self, wl):
        self.wl = wl
        self.kc, self.wn, self.Q = wl.kc(), wl.wn(), wl.Q()
        self.gc = wl.gc() if wl.ratio == 2 else None
        self.qI, self.wI = wl.qI(), wl.wI()
        self.derive = wl.keys == "derive"
        self.ki = None if self.derive else wl.ki_given()
        self.cos, self.sin = [_up(a) for a in __import__("csa2_synth").rope_table(wl.rope_rows)]
        self.gamma_c, self.gamma_ik = _up(wl.gamma_c()), _up(wl.gamma_ik())
        self.w_ik = _up(wl.w_ik()) if self.derive else None
        self.sink = _up(wl.sink())

    def span(self, name, b, p0, T):
        """request b's positions p0 .. p0+T-1 of a per-position tensor"""
        a = getattr(self, name)
        if name == "Q":
            return a[b][:, p0:p0 + T]
        if name == "ki":
            r = self.wl.ratio
            return a[b, p0 // r:(p0 + T) // r]
        return a[b, p0:p0 + T]

    def batch(self, name, bs, p0s, T):
        if getattr(self, name) is None:
            return None
        return _up(np.ascontiguousarray(np.stack([self.span(name, b, p, T)
                                                  for b, p in zip(bs, p0s)])))


def _forward_prefill(inp, cc, bs, p0s, T):
    """one csa2_forward over new positions p0s[i] .. p0s[i]+T-1 of requests bs, into
    caches cc (row i of the call = cache row i)"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    wl = inp.wl
    B = len(bs)
    idx = torch.full((B, T, 512), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    O = torch.zeros(B, wl.H, T, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, wl.H, T, dtype=torch.float32, device="cuda")
    ws = csa2.workspace(csa2.OP_FORWARD, B, T, wl.H, cc.stride)
    csa2.csa2_forward(_up(np.array(p0s, np.int32)), inp.batch("Q", bs, p0s, T),
                      inp.batch("qI", bs, p0s, T), inp.batch("wI", bs, p0s, T), inp.sink, inp.cos,
                      inp.sin, cc.z_codes, cc.z_scales, cc.ki_codes, cc.ki_scales, cc.w_codes,
                      cc.w_scale, idx, cnt, O, ws, kc=inp.batch("kc", bs, p0s, T),
                      gc=inp.batch("gc", bs, p0s, T), wn=inp.batch("wn", bs, p0s, T),
                      gamma_c=inp.gamma_c, w_ik=inp.w_ik, gamma_ik=inp.gamma_ik,
                      ki_given=inp.batch("ki", bs, p0s, T), lse=lse, ratio=wl.ratio,
                      z_format=wl.z_format)
    torch.cuda.synchronize()
    return _down(idx), _down(cnt), _down(O), _down(lse)


def _check_caches(cc, row, ref, n_ent, last_pos):
    """cache row `row` holds the oracle's entries below n_ent and the window rows of
    the positions the ring still holds (the last cap up to last_pos)"""
    for k in ("z_codes", "z_scales", "ki_codes", "ki_scales"):
        got = _down(getattr(cc, k))[row, :n_ent]
        assert np.array_equal(got, getattr(ref, k)[0, :n_ent]), k
    w_codes, w_scale = ref.window_full()
    pos = np.arange(max(0, last_pos + 1 - cc.cap), last_pos + 1)
    assert np.array_equal(_down(cc.w_codes)[row, pos % cc.cap], w_codes[pos])
    assert np.array_equal(_down(cc.w_scale)[row, pos % cc.cap], w_scale[pos])


def _check_rows(wl, ref, ts, g_idx, g_cnt, g_O, what):
    """rows at global positions ts (request of ref) against the oracle; g_* indexed like ts"""
    import oracle
    r = prefill_rows_parallel(ref, ts, want_scores=True)
    swaps = 0
    exp = r["O"].copy()
    for i, t in enumerate(ts):
        swaps += check_selection(g_idx[i], g_cnt[i], r["idx"][i], r["cnt"][i], r["S"][i])
        if not np.array_equal(g_idx[i], r["idx"][i]):
            exp[i] = oracle.attend(wl.Q_rows(ref.b, [t])[0], int(t), ref.w_codes[0],
                                   ref.w_scale[0], ref.cap, ref.z_codes[0], ref.z_scales[0],
                                   g_idx[i], int(g_cnt[i]), ref.sink, ref.cos, ref.sin,
                                   z_format=wl.z_format)[0]
    mx, rel = check_attention(g_O, exp, what)
    log(f"  {what}: rows={len(ts)} swaps={swaps} max|dO|={mx:.2e} rel={rel:.2e}")


CASES = [(0, 2, 0), (1, 1, 0), (1, 2, 1)]     # (workload recipe, ratio, z_format)


@pytest.mark.parametrize("cid,ratio,zf", CASES)
def test_prefill_two_chunks(dev, synth, cid, ratio, zf):
    """chunk 1 at positions 0..T1-1, chunk 2 at T1..T1+T2-1 over the same caches and a
    ring of exactly T1+127 slots (chunk 2's rows wrap onto positions it no longer
    needs); both chunks' rows and the caches against one oracle run over T1+T2"""
    from oracle.reference import PrefillReference
    T1, T2 = (700, 500) if ratio == 2 else (701, 499)
    wl = synth.workload(cid, T=T1 + T2, H=32, ratio=ratio, z_format=zf)
    log(f"two-chunk prefill: {wl.name} T1={T1} T2={T2}")
    inp = Inputs(wl)
    cc = Caches(wl, 1, (T1 + T2) // ratio, max(T1, T2) + 127)
    i1, c1, o1, _ = _forward_prefill(inp, cc, [0], [0], T1)
    i2, c2, o2, _ = _forward_prefill(inp, cc, [0], [T1], T2)
    ref = PrefillReference(wl)
    _check_caches(cc, 0, ref, (T1 + T2) // ratio, T1 + T2 - 1)
    rng = np.random.default_rng(11)
    loc1 = np.unique(np.concatenate([[0, 1, T1 - 1], rng.integers(0, T1, 20)]))
    loc2 = np.unique(np.concatenate([[0, 1, 2, T2 - 1], rng.integers(0, T2, 40)]))
    _check_rows(wl, ref, loc1, i1[0, loc1], c1[0, loc1], o1[0][:, loc1].transpose(1, 0, 2),
                "chunk 1")
    _check_rows(wl, ref, T1 + loc2, i2[0, loc2], c2[0, loc2], o2[0][:, loc2].transpose(1, 0, 2),
                "chunk 2")
    assert np.all(c2[0] == np.minimum(512, (T1 + np.arange(T2) + 1) // ratio))


@pytest.mark.parametrize("cid,ratio,zf", CASES)
def test_prefill_batched_offsets(dev, synth, cid, ratio, zf):
    """three requests in one call, new positions starting at 0, 200 and 1100 (each
    request's earlier positions were compressed and windowed by earlier calls)"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    from oracle.reference import PrefillReference
    T = 260
    p0s = [0, 200, 1100]
    T_full = max(p0s) + T
    wl = dataclasses.replace(synth.workload(cid, T=T_full, H=16, ratio=ratio, z_format=zf), B=3)
    log(f"batched prefill with offsets {p0s}: {wl.name}")
    inp = Inputs(wl)
    cc = Caches(wl, 3, T_full // ratio, T + 127)
    for b, p0 in enumerate(p0s):          # earlier positions, one request at a time
        if p0 == 0:
            continue
        sl = lambda t: t[b:b + 1]
        csa2.csa2_compress(_up(np.zeros(1, np.int32)), inp.batch("kc", [b], [0], p0),
                           inp.batch("gc", [b], [0], p0), inp.gamma_c, inp.w_ik, inp.gamma_ik,
                           inp.batch("ki", [b], [0], p0), inp.cos, inp.sin, sl(cc.z_codes),
                           sl(cc.z_scales), sl(cc.ki_codes), sl(cc.ki_scales), ratio=ratio,
                           z_format=zf)
        # the window rows the new positions need (one call must not wrap the ring)
        w0 = max(0, p0 - 127)
        csa2.csa2_encode_window(_up(np.array([w0], np.int32)),
                                inp.batch("wn", [b], [w0], p0 - w0), inp.cos, inp.sin,
                                sl(cc.w_codes), sl(cc.w_scale))
    torch.cuda.synchronize()
    g_idx, g_cnt, g_O, _ = _forward_prefill(inp, cc, [0, 1, 2], p0s, T)
    rng = np.random.default_rng(13)
    loc = np.unique(np.concatenate([[0, 1, T - 1], rng.integers(0, T, 24)]))
    for b, p0 in enumerate(p0s):
        ref = PrefillReference(wl, b)
        _check_caches(cc, b, ref, (p0 + T) // ratio, p0 + T - 1)
        assert np.all(g_cnt[b] == np.minimum(512, (p0 + np.arange(T) + 1) // ratio))
        _check_rows(wl, ref, p0 + loc, g_idx[b, loc], g_cnt[b, loc],
                    g_O[b][:, loc].transpose(1, 0, 2), f"request {b} (from {p0})")


@pytest.mark.parametrize("ratio", [2, 1])
def test_decode_forward_writes_window(dev, synth, ratio):
    """csa2_forward in decode form with wn: the call writes the new tokens' window rows
    (slots first overwritten with other bytes), then selects and attends"""
    import torch
    import csa2_harness
    import compressed_sparse_attention_csa2_amd as csa2
    import oracle
    from oracle.reference import DecodeReference
    wl = synth.decode_workload(B=3, Tq=6, n_entries=2600, H=32, keys="lognormal_dup",
                               ratio=ratio)
    log(f"decode forward with window rows: {wl.name}")
    run = csa2_harness.DecodeRun(wl)
    ring_c, ring_s = run.w_codes.clone(), run.w_scale.clone()
    slots = torch.tensor([(wl.q_pos0 + i) % wl.cap for i in range(wl.Tq)], device="cuda")
    run.w_codes[:, slots] = 0x33
    run.w_scale[:, slots] = 5.0
    wn_new = _up(np.ascontiguousarray(wl.wn()[:, -wl.Tq:]))
    csa2.csa2_forward(run.q_pos0, run.Q, run.qI, run.wI, run.sink, run.rope_cos, run.rope_sin,
                      run.z_codes, run.z_scales, run.ki_codes, run.ki_scales, run.w_codes,
                      run.w_scale, run.idx, run.cnt, run.O, run.ws, wn=wn_new,
                      n_entries=run.n_entries, lse=run.lse, ratio=ratio)
    torch.cuda.synchronize()
    assert torch.equal(run.w_codes, ring_c) and torch.equal(run.w_scale, ring_s)
    out = run.fetch()
    for b in range(wl.B):
        ref = DecodeReference(wl, b)
        r = ref.rows(np.arange(wl.Tq), want_scores=True)
        for i in range(wl.Tq):
            check_selection(out["idx"][b, i], out["cnt"][b, i], r["idx"][i], r["cnt"][i],
                            r["S"][i])
        exp = r["O"].copy()
        for i in range(wl.Tq):     # a boundary swap: judge attention on the GPU's selection
            if not np.array_equal(out["idx"][b, i], r["idx"][i]):
                ref._ensure_z(out["idx"][b, i])
                exp[i] = oracle.attend(wl.Q()[b][:, i, :], wl.q_pos0 + i, ref.w_codes,
                                       ref.w_scale, wl.cap, ref.z_codes, ref.z_scales,
                                       out["idx"][b, i], int(out["cnt"][b, i]), ref.sink,
                                       ref.cos, ref.sin)[0]
        mx, rel = check_attention(out["O"][b].transpose(1, 0, 2), exp, f"request {b}")
        log(f"  request {b}: max|dO|={mx:.2e} rel={rel:.2e}")


@pytest.mark.parametrize("ratio,zf", [(2, 0), (1, 0), (2, 1)])
def test_decode_over_prefill_caches(dev, synth, ratio, zf):
    """a decode call at position p over the caches a prefill left reproduces the
    prefill's row p: the same selection bit for bit, the output within tolerance of
    the prefill's and of the oracle's"""
    import torch
    import csa2_harness
    import compressed_sparse_attention_csa2_amd as csa2
    from oracle.reference import PrefillReference
    T = 1400
    wl = synth.workload(1, T=T, H=32, ratio=ratio, z_format=zf)
    log(f"decode over prefill caches: {wl.name}")
    run = csa2_harness.PrefillRun(wl)
    run.forward()
    torch.cuda.synchronize()
    P = np.array([T - 1, 1100, 1023, 700, 513, 3])
    ne = _up(np.array([T // ratio], np.int32))
    ref = PrefillReference(wl)
    ref.window_full()
    r = prefill_rows_parallel(ref, P, want_scores=True)
    for i, p in enumerate(P):
        sl = slice(int(p), int(p) + 1)
        Q = run.Q[:, :, sl].contiguous()
        qI, wI = run.qI[:, sl].contiguous(), run.wI[:, sl].contiguous()
        idx = torch.full((1, 1, 512), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((1, 1), -7, dtype=torch.int32, device="cuda")
        O = torch.zeros(1, wl.H, 1, 512, dtype=torch.bfloat16, device="cuda")
        ws = csa2.workspace(csa2.OP_FORWARD, 1, 1, wl.H, run.stride)
        csa2.csa2_forward(_up(np.array([p], np.int32)), Q, qI, wI, run.sink, run.rope_cos,
                          run.rope_sin, run.z_codes, run.z_scales, run.ki_codes, run.ki_scales,
                          run.w_codes, run.w_scale, idx, cnt, O, ws, n_entries=ne, ratio=ratio,
                          z_format=zf)
        torch.cuda.synchronize()
        d_idx, d_cnt = _down(idx)[0, 0], int(_down(cnt)[0, 0])
        p_idx, p_cnt = _down(run.idx[0, sl])[0], int(_down(run.cnt[0, sl])[0])
        assert d_cnt == p_cnt and np.array_equal(d_idx, p_idx), f"p={p}"
        check_selection(d_idx, d_cnt, r["idx"][i], r["cnt"][i], r["S"][i])
        d_O = _down(O)[0][:, 0]
        p_O = _down(run.O[0][:, sl].contiguous())[:, 0]
        from tests.parity import bf16_to_f64
        check_attention(d_O, bf16_to_f64(p_O), f"p={p} decode vs prefill")
        mx, rel = check_attention(d_O, r["O"][i], f"p={p} decode vs oracle")
        log(f"  p={p}: cnt={d_cnt} max|dO|={mx:.2e} rel={rel:.2e}")


def test_quant_index_query_bit_exact_full_size(dev, synth, orc):
    """the indexer's E4M3 query rows and folded weights for every (token, head) row of
    the 65,536-token workload, plus edge rows (zero, tiny, huge, exact ties, saturation),
    and rows whose largest element is 448, so that the quotient is the value itself and
    the hardware E4M3 conversion meets every rounding midpoint of the format (normal and
    subnormal, both signs) and the values one bf16 step to either side"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    wl = synth.workload(2)
    qI = wl.qI().reshape(-1, 32, 128)
    wI = wl.wI().reshape(-1, 32)
    rng = np.random.default_rng(29)
    edge = rng.standard_normal((8, 32, 128)).astype(np.float32)
    edge[0] = 0.0
    edge[1] *= 1e-30
    edge[2] *= 1e30
    edge[3] = np.round(edge[3] * 8) / 8
    edge[4, :, ::3] = 0.0
    edge[5] = np.ldexp(1.0, rng.integers(-20, 20, (32, 128))) * rng.choice([-1, 1], (32, 128))
    edge[6] = rng.choice([448.0, 464.0, 480.0, -448.0], (32, 128))
    edge[7] = np.exp(rng.standard_normal((32, 128)) * 4)
    # E4M3 midpoints: (1 + (2m + 1)/16) 2^e for normal codes, (k + 1/2) 2^-9 below 2^-6
    mids = [(1 + (2 * m + 1) / 16) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    mids += [(k + 0.5) * 2.0 ** -9 for k in range(8)]
    mids = np.array([v for v in mids if v < 464.0])
    vals = np.concatenate([mids, mids * (1 + 2.0 ** -7), mids * (1 - 2.0 ** -7)])
    vals = np.concatenate([vals, -vals])
    ties = np.zeros((2, 32, 128), np.float32)
    flat = np.resize(vals, 2 * 32 * 127).reshape(2, 32, 127)
    ties[:, :, 0] = 448.0
    ties[:, :, 1:] = flat
    qI = np.concatenate([qI, tc.bf16(edge), tc.bf16(ties)])
    wI = np.concatenate([wI, (rng.standard_normal((10, 32)) / 64).astype(np.float32)])
    rows = qI.shape[0] * 32
    log(f"csa2_quant_index_query: {rows} rows")
    q8 = torch.zeros(rows, 128, dtype=torch.uint8, device=dev)
    wq = torch.zeros(rows, dtype=torch.float32, device=dev)
    csa2.csa2_quant_index_query(_up(qI), _up(wI), q8, wq)
    torch.cuda.synchronize()
    g8, gw = _down(q8).reshape(-1, 32, 128), _down(wq).reshape(-1, 32)
    from tests.parity import parallel_map
    def one(t):
        o8, osq = orc.quant_index_query(qI[t])
        return (np.array_equal(g8[t], o8) and
                np.array_equal(gw[t], (wI[t] * osq).astype(np.float32)))
    ok = parallel_map(lambda ts: all(one(t) for t in ts),
                      np.array_split(np.arange(qI.shape[0]), 64))
    assert all(ok)
