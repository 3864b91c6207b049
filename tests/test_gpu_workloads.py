"""The five measured workloads at full size, in the launch configuration the
benchmark times (one csa2_forward), compared with the oracle on sampled rows.
Storage codes are compared in full where the oracle can produce them quickly."""
import numpy as np
import pytest

from tests.parity import check_attention, check_selection

pytestmark = pytest.mark.gpu


def log(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda"


def _attn_expected(wl, ref, b, rows_local, positions, g_idx, g_cnt, r, Qrows):
    """oracle attention on the GPU's selection where a boundary swap changed it"""
    import oracle
    exp = r["O"].copy()
    for i in range(len(rows_local)):
        if not np.array_equal(g_idx[i], r["idx"][i]):
            O, _, _ = oracle.attend(Qrows[i], int(positions[i]), ref.w_codes if ref.w_codes.ndim == 2 else ref.w_codes[0],
                                    ref.w_scale if ref.w_scale.ndim == 1 else ref.w_scale[0], wl.cap,
                                    ref.z_codes if ref.z_codes.ndim == 2 else ref.z_codes[0],
                                    ref.z_scales if ref.z_scales.ndim == 2 else ref.z_scales[0],
                                    g_idx[i], int(g_cnt[i]), ref.sink, ref.cos, ref.sin,
                                    z_format=wl.z_format)
            exp[i] = O
    return exp


def stratified_rows(T, nrows, seed):
    """nrows query rows of a T-token prefill: the first rows, the boundary where the
    selection starts (t = 1022, 1023), the last 32 rows (the heaviest), and the rest
    drawn evenly from 48 equal strata of [0, T)"""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 1021, 1022, 1023, 1024] + list(range(T - 32, T))
    per = max(1, -(-(nrows - len(fixed)) // 48))
    edges = np.linspace(0, T, 49).astype(np.int64)
    strata = [rng.integers(edges[i], edges[i + 1], per) for i in range(48)]
    return np.unique(np.concatenate([fixed] + strata))


@pytest.mark.parametrize("cid,nrows", [(1, 128), (2, 256)])
def test_prefill_workload(dev, synth, cid, nrows):
    import torch
    import csa2_harness
    from oracle.reference import PrefillReference
    from tests.parity import prefill_rows_parallel
    wl = synth.workload(cid)
    log(f"workload {cid}: {wl.name}")
    run = csa2_harness.PrefillRun(wl)
    run.forward()
    torch.cuda.synchronize()
    T = wl.Tq
    rows = stratified_rows(T, nrows, 100 + cid)
    assert len(rows) >= nrows * 0.9
    ti = torch.from_numpy(rows).cuda()
    g_idx = run.idx[0, ti].cpu().numpy()
    g_cnt = run.cnt[0, ti].cpu().numpy()
    g_O = csa2_harness.down(run.O[0][:, ti, :].contiguous()).transpose(1, 0, 2)
    zc, zs = csa2_harness.down(run.z_codes), csa2_harness.down(run.z_scales)
    kc, ks = csa2_harness.down(run.ki_codes), csa2_harness.down(run.ki_scales)
    wc, wsc = csa2_harness.down(run.w_codes), csa2_harness.down(run.w_scale)
    del run
    torch.cuda.empty_cache()
    ref = PrefillReference(wl)
    assert np.array_equal(zc, ref.z_codes) and np.array_equal(zs, ref.z_scales)
    assert np.array_equal(kc, ref.ki_codes) and np.array_equal(ks, ref.ki_scales)
    w_codes, w_scale = ref.window_full()
    assert np.array_equal(wc[0, :T], w_codes[:T]) and np.array_equal(wsc[0, :T], w_scale[:T])
    r = prefill_rows_parallel(ref, rows, want_scores=True)
    swaps = sum(check_selection(g_idx[i], g_cnt[i], r["idx"][i], r["cnt"][i], r["S"][i])
                for i in range(len(rows)))
    exp = _attn_expected(wl, ref, 0, rows, rows, g_idx, g_cnt, r, wl.Q_rows(0, rows))
    mx, rel = check_attention(g_O, exp, wl.name)
    log(f"  rows={len(rows)} swaps={swaps} max|dO|={mx:.2e} rel={rel:.2e}")


@pytest.mark.parametrize("cid,reqs,qrows,form", [
    (3, (0, 17, 33, 50, 77, 96, 111, 127), (0,), None),
    (4, (5, 12), (0, 1, 2, 3, 4, 5), None),
    (3, (0, 17, 50, 77, 111, 127), (0,), "ratio1_z16")])
def test_decode_workload(dev, synth, cid, reqs, qrows, form):
    """the measured decode shapes at full size; ratio1_z16: the B=128 decode in the
    decoder layers' form as the benchmark runs it (131,072 entries per request at
    compression ratio 1, rows in the pages' 288-byte format)"""
    import dataclasses
    import torch
    import csa2_harness
    from oracle.reference import DecodeReference
    from tests.parity import parallel_map
    wl = synth.workload(cid)
    if form == "ratio1_z16":
        wl = dataclasses.replace(wl, n_entries=wl.q_pos0 + wl.Tq, ratio=1, z_format=1,
                                 name=wl.name + " ratio 1 Z per-16 E4M3")
    log(f"workload {cid}: {wl.name}")
    run = csa2_harness.DecodeRun(wl)
    run.forward()
    torch.cuda.synchronize()
    out = run.fetch()
    del run
    torch.cuda.empty_cache()
    q = np.array(qrows)

    def one(b):
        ref = DecodeReference(wl, b)
        r = ref.rows(q, want_scores=True)
        swaps = sum(check_selection(out["idx"][b, i], out["cnt"][b, i], r["idx"][k],
                                    r["cnt"][k], r["S"][k]) for k, i in enumerate(q))
        ref._ensure_z(out["idx"][b, q].reshape(-1))
        Qr = wl.Q()[b][:, q, :].transpose(1, 0, 2)
        exp = _attn_expected(wl, ref, b, q, wl.q_pos0 + q, out["idx"][b, q], out["cnt"][b, q],
                             r, Qr)
        got = out["O"][b][:, q, :].transpose(1, 0, 2)
        mx, rel = check_attention(got, exp, f"{wl.name} request {b}")
        return f"  request {b}: swaps={swaps} max|dO|={mx:.2e} rel={rel:.2e}"

    for line in parallel_map(one, reqs, threads=min(len(reqs), 8)):
        log(line)
