"""Pins of the oracle's hierarchical candidate pool and Reindex selection (no GPU).

Pages: "Inside DeepSeek V4.1" (the Hierarchical Sparse Indexer paragraph) and
"Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache" (section
"Hierarchical indexing bounds the later searches"): blocks of 8 entries ranked
by their largest score, 2,048 blocks kept (at most 16,384 candidates, about 61
times fewer than a scan of 10^6), the newest block always kept; Reindex layers
pick their own top 512 inside the pool.

Pins: the pool against a pairwise-count formulation of "the keep-1 best other
blocks" on small cases with ties; its size bounds and the page's 61x figure;
the newest block kept even when it scores lowest; Reindex with the Full
layer's own query returns the Full layer's top 512 (each selected entry's block
has a key at or above the 512th score, so at most 512 blocks beat it); with at
most 2,048 blocks the pool is everything and Reindex equals a full top 512.
"""
import numpy as np
import pytest

rng = np.random.default_rng(31)


def pairwise_pool(S, n, block, keep):
    """block b (not the newest) is kept iff fewer than keep-1 other non-newest
    blocks beat it (larger key, or equal key and smaller index)"""
    nb = (n + block - 1) // block
    if nb <= keep:
        return list(range(nb))
    key = [max(S[b * block:min(n, (b + 1) * block)]) for b in range(nb - 1)]
    out = []
    for b in range(nb - 1):
        beat = sum(1 for c in range(nb - 1) if key[c] > key[b] or (key[c] == key[b] and c < b))
        if beat < keep - 1:
            out.append(b)
    return out + [nb - 1]


@pytest.mark.parametrize("n,block,keep", [(1, 8, 5), (8, 8, 5), (40, 8, 5), (41, 8, 5),
                                          (300, 8, 5), (301, 8, 7), (1000, 8, 16), (257, 4, 9)])
def test_pool_matches_pairwise_definition_with_ties(orc, n, block, keep):
    S = (rng.integers(0, 12, n) * 0.25).astype(np.float32)     # many equal scores
    got = orc.pool_blocks(S, n, block, keep).tolist()
    assert got == pairwise_pool(S.tolist(), n, block, keep)
    assert got == sorted(got)


def test_pool_size_and_page_ratio(orc):
    n = 1_000_000
    S = rng.standard_normal(n).astype(np.float32)
    pool = orc.pool_blocks(S, n)
    cand = orc.pool_entries(pool, n)
    assert len(pool) == 2048 and len(cand) == 16384
    assert abs(n / len(cand) - 61.04) < 0.01          # the pages' "about 61 times"
    assert pool[-1] == (n - 1) // 8                    # the newest block


def test_pool_keeps_newest_block_when_it_scores_lowest(orc):
    n = 20_003                                         # newest block holds entries 20000..20002
    S = rng.uniform(1.0, 2.0, n).astype(np.float32)
    S[20_000:] = -5.0
    pool = orc.pool_blocks(S, n)
    assert pool[-1] == 2500 and len(pool) == 2048
    keys = np.array([S[b * 8:(b + 1) * 8].max() for b in range(2500)])
    thr = np.sort(keys)[::-1][2046]
    assert np.all(keys[pool[:-1]] >= thr)


def _index_setup(orc, N, seed):
    r = np.random.default_rng(seed)
    kc, ks = orc.fp4_encode(r.standard_normal((N, 128)).astype(np.float32))
    q = (r.standard_normal((32, 128))).astype(np.float32)
    u = np.asarray(q, np.float32).view(np.uint32).astype(np.uint64)
    q16 = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    q8, sq = orc.quant_index_query(q16)
    w = (r.standard_normal(32) / 64).astype(np.float32)
    return kc, ks, q8, sq, w


def test_reindex_with_full_query_returns_full_selection(orc):
    N = 20_000                                         # 2,500 blocks: the pool is a real subset
    kc, ks, q8, sq, w = _index_setup(orc, N, 5)
    for n in (N, 18_001, 16_390):
        S = orc.index_scores(q8, sq, w, kc, ks, n)
        full_idx, full_cnt = orc.topk(S, n)
        pool = orc.pool_blocks(S, n)
        assert len(pool) == 2048
        idx, cnt, cand, _ = orc.reindex_topk(q8, sq, w, kc, ks, n, pool)
        assert cnt == full_cnt == 512
        assert np.array_equal(idx, full_idx)


def test_reindex_over_whole_pool_is_full_topk_of_new_query(orc):
    N = 9_000                                          # 1,125 blocks <= 2,048
    kc, ks, q8, sq, w = _index_setup(orc, N, 6)
    _, _, q8b, sqb, wb = _index_setup(orc, N, 7)       # another layer's query
    S = orc.index_scores(q8, sq, w, kc, ks, N)
    pool = orc.pool_blocks(S, N)
    assert np.array_equal(pool, np.arange(1125))
    idx, cnt, cand, _ = orc.reindex_topk(q8b, sqb, wb, kc, ks, N, pool)
    Sb = orc.index_scores(q8b, sqb, wb, kc, ks, N)
    ref_idx, ref_cnt = orc.topk(Sb, N)
    assert cnt == ref_cnt and np.array_equal(idx, ref_idx)
