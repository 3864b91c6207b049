"""csa2_index_topk_noalloc (the library's own scratch array, no workspace) against
csa2_index_topk (caller's workspace) on the same inputs, bit for bit, over
calls in a row that shrink: few long rows (score rows then selection), rows
cut into segments (the fused kernel with its per-row arrival counters, which
the call must clear), and one small fused call."""
import numpy as np
import pytest

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


def _case(orc, rng, B, Tq, N, ratio):
    """device tensors of B requests x Tq queries over N random FP4 index keys"""
    import csa2_harness
    import tests.test_oracle_compress as tc
    up = csa2_harness.up
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.zeros((B, N, 4), np.uint8)
    for b in range(B):
        kc[b], ks[b] = orc.fp4_encode(rng.standard_normal((N, 128)).astype(np.float32))
    qI = tc.bf16(rng.standard_normal((B, Tq, 32, 128)).astype(np.float32))
    wI = (rng.standard_normal((B, Tq, 32)) / 64).astype(np.float32)
    q0 = np.array([ratio * N - Tq - 3 * b for b in range(B)], np.int32)
    ne = np.array([N - 7 * b for b in range(B)], np.int32)
    return dict(q0=up(q0), ne=up(ne), qI=up(qI), wI=up(wI), kc=up(kc), ks=up(ks))


def _both(c, B, Tq, ratio):
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    N = c["kc"].shape[1]
    out = []
    for noalloc in (False, True):
        idx = torch.full((B, Tq, 512), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Tq), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            csa2.csa2_index_topk_noalloc(c["q0"], c["ne"], c["qI"], c["wI"], c["kc"], c["ks"],
                                         idx, cnt, ratio=ratio)
        else:
            ws = csa2.workspace(csa2.OP_INDEX_TOPK, B, Tq, 64, N)
            csa2.csa2_index_topk(c["q0"], c["ne"], c["qI"], c["wI"], c["kc"], c["ks"], idx, cnt,
                                 ws, ratio=ratio)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), cnt.cpu().numpy()))
    return out


def test_noalloc_matches_workspace_calls(dev, orc):
    import compressed_sparse_attention_csa2_amd as csa2
    rng = np.random.default_rng(41)
    # call 1: few long rows (score rows in the scratch, then the selection pass)
    # call 2: two rows cut into segments (arrival counters in the scratch)
    # call 3: a small call, one segment per row
    for B, Tq, N, ratio in ((4, 6, 20000, 2), (2, 1, 12000, 1), (1, 5, 3000, 2)):
        need = csa2.workspace_size(csa2.OP_INDEX_TOPK, B, Tq, 64, N)
        assert need <= csa2.NOALLOC_SCRATCH_BYTES
        log(f"index_topk_noalloc: B={B} Tq={Tq} N={N} ratio={ratio} (scratch {need} bytes)")
        c = _case(orc, rng, B, Tq, N, ratio)
        (ia, ca), (ib, cb) = _both(c, B, Tq, ratio)
        assert np.array_equal(ca, cb) and np.array_equal(ia, ib)
        assert np.all(ca == np.minimum(512, ca)) and np.all(ca > 0)


def test_noalloc_rejects_sizes_beyond_its_scratch(dev):
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    B, Tq, N = 1, 65536, 32768            # 277 MB of workspace
    assert csa2.workspace_size(csa2.OP_INDEX_TOPK, B, Tq, 64, N) > csa2.NOALLOC_SCRATCH_BYTES
    z = lambda *s, dt=torch.uint8: torch.zeros(*s, dtype=dt, device="cuda")
    with pytest.raises(csa2.CSA2Error, match="scratch"):
        csa2.csa2_index_topk_noalloc(z(B, dt=torch.int32), z(B, dt=torch.int32),
                                     z(B, Tq, 32, 128, dt=torch.bfloat16),
                                     z(B, Tq, 32, dt=torch.float32), z(B, N, 64), z(B, N, 4),
                                     z(B, Tq, 512, dt=torch.int32), z(B, Tq, dt=torch.int32))
