"""GPU parity of the hierarchical candidate pool and the Reindex selection
(csa2_index_pool, csa2_reindex_topk) through the C ABI, against the oracle.

Four requests over a 20,000-entry index-key cache with 2% of the entries
copying earlier entries' bytes (exact score ties), queried at positions where
the rows see 20,000 / about 18,000 entries (more than 2,048 blocks of 8: the
pool is a real subset, the newest block partial), about 9,000 entries (every
block in the pool) and about 3,000 entries (fewer than 512 blocks: Reindex
selects from a list shorter than the one-block-per-row kernel's sample size).  Checks: the Full selection as csa2_index_topk; the
pool block sets (boundary swaps between blocks whose oracle keys agree to
1e-5 relative, as for the top-512); the newest block present; Reindex with
another layer's query over the oracle's pool against the oracle's Reindex
selection; Reindex with the Full layer's own query over the GPU's pool equal
to the GPU's Full selection, bit for bit.
"""
import numpy as np
import pytest

from tests.parity import check_selection, SWAP_REL

pytestmark = pytest.mark.gpu


def log(*a):
    print("[gpu]", *a, flush=True)


def check_pool(g_pool, g_cnt, o_pool, S, n):
    """one row; returns the number of boundary swaps"""
    o_cnt = len(o_pool)
    assert int(g_cnt) == o_cnt, f"pool size {g_cnt} != oracle {o_cnt}"
    g = np.asarray(g_pool[:o_cnt])
    assert np.all(g_pool[o_cnt:] == -1)
    assert np.all(np.diff(g) > 0), "pool must be ascending"
    nb = (n + 7) // 8
    assert g[-1] == nb - 1, "the newest block must be in the pool"
    a, b = set(g.tolist()), set(o_pool.tolist())
    if a == b:
        return 0
    only_g, only_o = sorted(a - b), sorted(b - a)
    assert len(only_g) == len(only_o)
    keys = np.array([S[k * 8:min(n, k * 8 + 8)].max() for k in only_g + only_o], np.float64)
    spread, scale = keys.max() - keys.min(), np.abs(keys).max()
    assert spread <= SWAP_REL * scale, f"non-boundary pool swap: {only_g[:4]} vs {only_o[:4]}"
    return len(only_g)


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("ratio", [2, 1])
def test_pool_and_reindex_match_oracle(ratio):
    """ratio 1 (one entry per position, as in the decoder layers that use the pool):
    the same rows at positions that see the same entry counts"""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_csa2_amd as csa2
    import oracle
    from csa2_harness import up, down

    rng = np.random.default_rng(41)
    B, Tq, N = 4, 3, 20_000
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    for b in range(B):
        kc[b], ks[b] = oracle.fp4_encode(rng.standard_normal((N, 128)).astype(np.float32))
        dup = rng.random(N) < 0.02
        dup[0] = False
        src = (rng.random(N) * np.arange(N)).astype(np.int64)
        kc[b][dup], ks[b][dup] = kc[b][src[dup]], ks[b][src[dup]]
    qI = _bf16(rng.standard_normal((B, Tq, 32, 128)))
    wI = (rng.standard_normal((B, Tq, 32)) / 64).astype(np.float32)
    qI2 = _bf16(rng.standard_normal((B, Tq, 32, 128)))
    wI2 = (rng.standard_normal((B, Tq, 32)) / 64).astype(np.float32)
    q_pos0 = np.array([ratio * N, ratio * 18_001 - 1, ratio * 9_000, ratio * 3_000], np.int32)
    n_entries = np.full(B, N, np.int32)
    log(f"csa2_index_pool / csa2_reindex_topk: B={B} Tq={Tq} N={N} ratio={ratio}")

    g = dict(q0=up(q_pos0), ne=up(n_entries), kc=up(kc), ks=up(ks))
    idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    pool = torch.full((B, Tq, 2048), -7, dtype=torch.int32, device="cuda")
    pcnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(csa2.OP_INDEX_POOL, B, Tq, 64, N)
    csa2.csa2_index_pool(g["q0"], g["ne"], up(qI), up(wI), g["kc"], g["ks"], idx, cnt, pool, pcnt,
                         ws, ratio=ratio)
    # reindex with the Full query over the GPU pool; with another query over the oracle pool
    idx_same = torch.full_like(idx, -7)
    cnt_same = torch.full_like(cnt, -7)
    wsr = csa2.workspace(csa2.OP_REINDEX, B, Tq, 64, N)
    csa2.csa2_reindex_topk(g["q0"], g["ne"], up(qI), up(wI), g["kc"], g["ks"], pool, pcnt,
                           idx_same, cnt_same, wsr, ratio=ratio)
    o_pools = np.full((B, Tq, 2048), -1, np.int32)
    o_pcnt = np.zeros((B, Tq), np.int32)
    ref = {}
    for b in range(B):
        for i in range(Tq):
            n = min((int(q_pos0[b]) + i + 1) // ratio, N)
            q8, sq = oracle.quant_index_query(qI[b, i])
            S = oracle.index_scores(q8, sq, wI[b, i], kc[b], ks[b], n)
            p = oracle.pool_blocks(S, n)
            o_pools[b, i, :len(p)] = p
            o_pcnt[b, i] = len(p)
            ref[b, i] = (n, S, p) + oracle.topk(S, n)
    idx2 = torch.full_like(idx, -7)
    cnt2 = torch.full_like(cnt, -7)
    csa2.csa2_reindex_topk(g["q0"], g["ne"], up(qI2), up(wI2), g["kc"], g["ks"], up(o_pools),
                           up(o_pcnt), idx2, cnt2, wsr, ratio=ratio)
    torch.cuda.synchronize()
    gi, gc_, gp, gpc = down(idx), down(cnt), down(pool), down(pcnt)
    gis, gcs, gi2, gc2 = down(idx_same), down(cnt_same), down(idx2), down(cnt2)

    swaps = pswaps = rswaps = 0
    for b in range(B):
        for i in range(Tq):
            n, S, p, r_idx, r_cnt = ref[b, i]
            swaps += check_selection(gi[b, i], gc_[b, i], r_idx, r_cnt, S)
            pswaps += check_pool(gp[b, i], gpc[b, i], p, S, n)
            assert gcs[b, i] == gc_[b, i] and np.array_equal(gis[b, i], gi[b, i]), \
                f"reindex with the Full query != Full selection at {(b, i)}"
            q8b, sqb = oracle.quant_index_query(qI2[b, i])
            o_idx, o_cnt, cand, Sc = oracle.reindex_topk(q8b, sqb, wI2[b, i], kc[b], ks[b], n, p)
            full = np.full(n, np.nan)
            full[cand] = Sc
            rswaps += check_selection(gi2[b, i], gc2[b, i], o_idx, o_cnt, full)
    log(f"  rows={B * Tq} topk swaps={swaps} pool swaps={pswaps} reindex swaps={rswaps}")


def test_pool_many_blocks_skewed_keys():
    """12,500 blocks per row (six times the pool): request 0 with log-normal key norms;
    request 1 with 1,024 blocks on a regular lattice holding keys far above all others
    (a pool of those plus the best of the rest).  Both against the oracle."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_csa2_amd as csa2
    import oracle
    from csa2_harness import up, down

    rng = np.random.default_rng(43)
    B, Tq, N = 2, 1, 100_000
    nb = (N + 7) // 8
    m = nb - 1
    sampled = np.unique(((np.arange(1024, dtype=np.int64)) * m) >> 10)
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    x0 = rng.standard_normal((N, 128)) * np.exp(rng.standard_normal((N, 1)))
    kc[0], ks[0] = oracle.fp4_encode(x0.astype(np.float32))
    x1 = rng.standard_normal((N, 128))
    big = np.zeros(N, bool)
    for k in sampled:
        big[8 * k:8 * k + 8] = True
    x1[big] *= 16.0
    kc[1], ks[1] = oracle.fp4_encode(x1.astype(np.float32))
    qI = _bf16(rng.standard_normal((B, Tq, 32, 128)))
    wI = (np.abs(rng.standard_normal((B, Tq, 32))) / 64).astype(np.float32)   # S grows with |k|
    q_pos0 = np.full(B, N - 1, np.int32)                # ratio 1: every entry visible
    log(f"pool over many blocks: B={B} N={N} blocks={nb}")
    idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    pool = torch.full((B, Tq, 2048), -7, dtype=torch.int32, device="cuda")
    pcnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(csa2.OP_INDEX_POOL, B, Tq, 64, N)
    csa2.csa2_index_pool(up(q_pos0), up(np.full(B, N, np.int32)), up(qI), up(wI), up(kc), up(ks),
                         idx, cnt, pool, pcnt, ws, ratio=1)
    torch.cuda.synchronize()
    gp, gpc, gi, gc_ = down(pool), down(pcnt), down(idx), down(cnt)
    for b in range(B):
        q8, sq = oracle.quant_index_query(qI[b, 0])
        S = oracle.index_scores(q8, sq, wI[b, 0], kc[b], ks[b], N)
        p = oracle.pool_blocks(S, N)
        if b == 1:     # the construction: the lattice blocks hold the largest keys
            keys = np.array([S[8 * k:8 * k + 8].max() for k in range(m)])
            assert np.all(np.sort(keys)[::-1][:len(sampled)] >= keys[~np.isin(np.arange(m), sampled)].max())
        swaps = check_pool(gp[b, 0], gpc[b, 0], p, S, N)
        r_idx, r_cnt = oracle.topk(S, N)
        swaps += check_selection(gi[b, 0], gc_[b, 0], r_idx, r_cnt, S)
        log(f"  request {b}: pool {len(p)} blocks, swaps {swaps}")


@pytest.mark.parametrize("ratio", [2, 1])
def test_pool_verify_decode_full_size(ratio):
    """the verify-decode shape as the benchmark runs it (B=16 x 6 queries at 1,048,570..,
    log-normal keys with 1% exact duplicates; 524,288 entries at ratio 2, 1,048,576 at
    ratio 1): request 5, query rows 0 and 5 -- Full selection, pool and a Reindex
    layer's selection against the oracle"""
    import dataclasses
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_csa2_amd as csa2
    import csa2_synth as synth
    import oracle
    from csa2_harness import up, down
    from oracle.reference import DecodeReference
    wl = synth.workload(4)
    if ratio == 1:
        wl = dataclasses.replace(wl, n_entries=wl.q_pos0 + wl.Tq, ratio=1)
    B, Tq, N = wl.B, wl.Tq, wl.n_entries
    log(f"pool at the verify-decode shape: ratio {ratio}, {N} entries")
    kc = torch.zeros(B, N, 64, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, N, 4, dtype=torch.uint8, device="cuda")
    for b in range(B):
        for j0 in range(0, N, 1 << 16):
            n = min(1 << 16, N - j0)
            csa2.csa2_encode_fp4_rows(up(wl.ki_rows(b, j0, n)), kc[b, j0:j0 + n].view(n, 64),
                                      ks[b, j0:j0 + n].view(n, 4))
    qI2 = synth.normal(wl.seed, 901, (B, Tq, 32, 128))
    wI2 = synth.normal(wl.seed, 902, (B, Tq, 32), mul=1.0 / 64.0, dtype="f32")
    q0 = torch.full((B,), wl.q_pos0, dtype=torch.int32, device="cuda")
    ne = torch.full((B,), N, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    pool = torch.full((B, Tq, 2048), -7, dtype=torch.int32, device="cuda")
    pcnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
    idx2, cnt2 = torch.full_like(idx, -7), torch.full_like(cnt, -7)
    csa2.csa2_index_pool(q0, ne, up(wl.qI()), up(wl.wI()), kc, ks, idx, cnt, pool, pcnt,
                         csa2.workspace(csa2.OP_INDEX_POOL, B, Tq, 64, N), ratio=ratio)
    csa2.csa2_reindex_topk(q0, ne, up(qI2), up(wI2), kc, ks, pool, pcnt, idx2, cnt2,
                           csa2.workspace(csa2.OP_REINDEX, B, Tq, 64, N), ratio=ratio)
    torch.cuda.synchronize()
    gi, gc_, gp, gpc, gi2, gc2 = (down(x) for x in (idx, cnt, pool, pcnt, idx2, cnt2))
    del kc, ks
    torch.cuda.empty_cache()
    b = 5
    ref = DecodeReference(wl, b)
    for i in (0, 5):
        n = min((wl.q_pos0 + i + 1) // ratio, N)
        q8, sq = oracle.quant_index_query(wl.qI()[b, i])
        S = oracle.index_scores(q8, sq, wl.wI()[b, i], ref.ki_codes, ref.ki_scales, n)
        r_idx, r_cnt = oracle.topk(S, n)
        swaps = check_selection(gi[b, i], gc_[b, i], r_idx, r_cnt, S)
        p = oracle.pool_blocks(S, n)
        pswaps = check_pool(gp[b, i], gpc[b, i], p, S, n)
        q8b, sqb = oracle.quant_index_query(qI2[b, i])
        o_idx, o_cnt, cand, Sc = oracle.reindex_topk(q8b, sqb, wI2[b, i], ref.ki_codes,
                                                     ref.ki_scales, n, gp[b, i][:int(gpc[b, i])])
        full = np.full(n, np.nan)
        full[cand] = Sc
        rswaps = check_selection(gi2[b, i], gc2[b, i], o_idx, o_cnt, full)
        log(f"  request {b} row {i}: n={n} topk swaps={swaps} pool swaps={pswaps} "
            f"reindex swaps={rswaps}")
