"""GPU parity of the decode selection without score rows (single-token query rows over
caches of at least 16,384 entries): a sampled threshold, a scan that keeps only the keys
at or above it in per-chunk slots, and a cut of those, with an exact fallback that scores
the row again when the sample misjudges. Every path against the oracle's top-512
("DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", top-k equation; ties:
the smaller entry)."""
import numpy as np
import pytest

from tests.parity import check_selection

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


N = 40_000                 # cache rows per request (the stride): above 16,384
CHUNK = 2048               # entries a scan wave covers; 512 candidate slots each


def _sample_threshold_range(S, n):
    """the keys the sampled threshold can take: between the sample's ks-th and
    (ks + ks/4)-th largest score of 1,024 entries spread over the row in 256 runs
    of four consecutive entries (each run starting at a multiple of four)"""
    i = np.arange(1024, dtype=np.int64)
    pos = ((((i >> 2) * n) >> 8) & ~np.int64(3)) + (i & 3)
    smp = np.sort(S[pos])[::-1]
    ks = (2048 * 1024 + n - 1) // n
    return smp[ks - 1], smp[ks + ks // 4 - 1]


def test_decode_selection_paths(dev, orc):
    """rows on every path: sampled and filtered (with 2% exact duplicate keys, so equal
    scores meet at the cut), at most 512 entries (all taken), 513..16,383 entries (the
    fallback), every key identical (the first chunk's slots overflow: fallback; ties keep
    the first 512 entries), the large scores only at 100 sampled entries (fewer than 512
    reach the threshold: fallback), and 1,500 large scores in one chunk (its slots
    overflow: fallback)"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(2024)
    ne = np.array([N, 300, 9000, N, N, N, 17_000], np.int32)
    B = len(ne)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    kpre = rng.standard_normal((B, N, 128))
    dup = rng.random(N) < 0.02                          # request 0: copies of earlier rows
    src = np.maximum(np.arange(N) - 1 - rng.integers(0, 50, N), 0)
    kpre[0][dup] = kpre[0][src[dup]]
    kpre[3] = kpre[3][:1]                               # request 3: one key everywhere
    n4 = int(ne[4])
    hot = ((((np.arange(100) * 10) >> 2) * n4) >> 8 & ~3) + (np.arange(100) * 10 & 3)   # request 4: 100 sampled entries
    kpre[4][hot] = 6.0 * u
    kpre[5][4096:5596] += 3.0 * u                       # request 5: a run inside chunk 2
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    for b in range(B):
        kc[b], ks[b] = orc.fp4_encode(kpre[b].astype(np.float32))
    qpre = rng.standard_normal((B, 1, 32, 128))
    qpre[4] = 4.0 * u + 0.3 * rng.standard_normal((1, 32, 128))
    qpre[5] = 4.0 * u + 0.3 * rng.standard_normal((1, 32, 128))
    qI = tc.bf16(qpre.astype(np.float32))
    wI = (rng.standard_normal((B, 1, 32)) / 64).astype(np.float32)
    wI[4:6] = np.abs(wI[4:6])
    q0 = np.full(B, 2 * N, np.int32)                     # every stored entry is a candidate
    log(f"decode selection paths: B={B} Tq=1 stride={N} rows={ne.tolist()}")
    idx = torch.full((B, 1, 512), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, 1), -7, dtype=torch.int32, device=dev)
    csa2.csa2_index_topk(_up(q0), _up(ne), _up(qI), _up(wI), _up(kc), _up(ks), idx, cnt,
                         csa2.workspace(csa2.OP_INDEX_TOPK, B, 1, 64, N))
    torch.cuda.synchronize()
    gi, gc_ = _down(idx), _down(cnt)
    for b in range(B):
        n = int(ne[b])
        q8, sq = orc.quant_index_query(qI[b, 0])
        S = orc.index_scores(q8, sq, wI[b, 0], kc[b], ks[b], n)
        r_idx, r_cnt = orc.topk(S, n)
        swaps = check_selection(gi[b, 0], gc_[b, 0], r_idx, r_cnt, S)
        log(f"  request {b}: n={n} swaps={swaps}")
        if b == 3:
            assert np.array_equal(gi[b, 0], np.arange(512)), "ties: the first 512 entries"
        if b in (0, 4, 5):
            hi_th, lo_th = _sample_threshold_range(S, n)
        if b == 0:
            # filtered: at least 512 reach any threshold the sample can give, no chunk overflows
            assert np.count_nonzero(S >= hi_th) >= 512
            per_chunk = [np.count_nonzero(S[c:c + CHUNK] >= lo_th) for c in range(0, n, CHUNK)]
            assert max(per_chunk) <= 512
            assert len(np.unique(S[r_idx[:r_cnt]])) < r_cnt, "equal scores among the selected"
        if b == 4:
            # the construction does what it is for: fewer than 512 reach the threshold
            assert np.count_nonzero(S >= lo_th) < 512
        if b == 5:
            # more than a chunk's 512 slots reach the threshold in chunk 2
            assert np.count_nonzero(S[2 * CHUNK:3 * CHUNK] >= hi_th) > 512


def test_decode_selection_in_forward_matches_two_pass_scores(dev, orc):
    """csa2_forward's decode selection (no score rows) equals the top-512 of
    csa2_index_scores' score rows on the same caches, bit for bit (both take the same
    fp32 scores), on 24 requests of mixed lengths at ratio 1 and 2"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    import tests.test_oracle_compress as tc
    rng = np.random.default_rng(99)
    B = 24
    for ratio in (2, 1):
        ne = rng.integers(16_000, N + 1, B).astype(np.int32)
        ne[:3] = [N, 20_000, 16_384]
        kc = np.zeros((B, N, 64), np.uint8)
        ks = np.zeros((B, N, 4), np.uint8)
        base_c, base_s = orc.fp4_encode(rng.standard_normal((N, 128)).astype(np.float32))
        for b in range(B):
            perm = rng.permutation(N)
            kc[b], ks[b] = base_c[perm], base_s[perm]
        qI = tc.bf16(rng.standard_normal((B, 1, 32, 128)).astype(np.float32))
        wI = (rng.standard_normal((B, 1, 32)) / 64).astype(np.float32)
        q0 = (ne.astype(np.int64) * ratio + 5).astype(np.int32)
        log(f"decode selection vs score rows: ratio={ratio} B={B} stride={N}")
        idx = torch.full((B, 1, 512), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((B, 1), -7, dtype=torch.int32, device=dev)
        csa2.csa2_index_topk(_up(q0), _up(ne), _up(qI), _up(wI), _up(kc), _up(ks), idx, cnt,
                             csa2.workspace(csa2.OP_INDEX_TOPK, B, 1, 64, N), ratio=ratio)
        S = torch.full((B, 1, N), float("nan"), dtype=torch.float32, device=dev)
        csa2.csa2_index_scores(_up(q0), _up(ne), _up(qI), _up(wI), _up(kc), _up(ks), S,
                               csa2.workspace(csa2.OP_INDEX_SCORES, B, 1, 64, N), ratio=ratio)
        torch.cuda.synchronize()
        gi, gc_, gS = _down(idx), _down(cnt), _down(S)
        for b in range(B):
            n = int(ne[b])
            r_idx, r_cnt = orc.topk(gS[b, 0, :n], n)
            assert int(gc_[b, 0]) == r_cnt
            assert np.array_equal(gi[b, 0], r_idx), f"request {b}"
