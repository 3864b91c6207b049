"""The C ABI on the CPU: the library loads, exports every declared symbol, sizes its
workspace, and rejects bad arguments before launching anything (no GPU needed:
every call here fails validation, so no HIP work is ever enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import compressed_sparse_attention_csa2_amd as csa2
    return csa2.lib()


def declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    return sorted(set(re.findall(r"^\s*(?:csa2_status|size_t|const char\*|int)\s+(csa2_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert L.csa2_abi_version() == 3
    for s in range(7):
        assert L.csa2_status_string(s)


def test_workspace_sizes(L):
    import compressed_sparse_attention_csa2_amd as csa2
    ws = csa2.workspace_size
    # the selection is fused into the scoring: no score rows, only the quantised
    # queries (4,224 bytes per query row) -- and segment winners when rows are few
    assert 65536 * 4224 <= ws(csa2.OP_INDEX_TOPK, 1, 65536, 64, 32768) < 65536 * 4224 + 4096
    # single-token rows over long caches (decode): no score rows, only the kept
    # candidates (512 slots of key and entry per 2,048 entries: 2 bytes an entry)
    assert 128 * 65536 * 2 <= ws(csa2.OP_INDEX_TOPK, 128, 1, 64, 65536) < 128 * 65536 * 2 + 2**20
    # up to eight tokens a request (verify): no score rows either (128 slots per
    # 2,048 entries at this length)
    assert ws(csa2.OP_INDEX_TOPK, 16, 6, 64, 524288) < 96 * 524288 * 4 // 4
    # many single-token rows stay fused: segment winners only
    assert ws(csa2.OP_INDEX_TOPK, 2048, 1, 64, 8192) < 2048 * 8192 * 4 // 4
    assert ws(csa2.OP_INDEX_TOPK, 3, 6, 64, 2600) <= 18 * (4224 + 16) + 4096
    assert ws(csa2.OP_INDEX_SCORES, 1, 65536, 64, 32768) < 65536 * 4224 + 4096
    assert ws(csa2.OP_FORWARD, 1, 256, 16, 128) > 0
    assert ws(csa2.OP_FORWARD, 1, 256, 17, 128) == 0          # heads not a multiple of 16
    assert ws(csa2.OP_FORWARD, 0, 256, 16, 128) == 0
    # a prefill: one split (no partials); the compressed rows re-encoded as E4M3
    # rows with an fp32 scale (512 + 4 bytes per entry), each 256-byte aligned
    assert ws(csa2.OP_SPARSE_ATTN, 1, 65536, 64, 32768) == 32768 * 512 + 32768 * 4
    # decode: a query's rows split over blocks below 128 queries (256 for the kernel
    # over the pages' 288-byte rows): partials, sized for either kernel
    assert ws(csa2.OP_SPARSE_ATTN, 128, 1, 64, 65536) > 0
    assert ws(csa2.OP_SPARSE_ATTN, 256, 1, 64, 65536) == 0
    # decode gathers each entry less than four times on average: no re-encoding
    assert ws(csa2.OP_SPARSE_ATTN, 128, 1, 64, 65536) < 128 * 65536 * 516
    assert ws(csa2.OP_SPARSE_ATTN, 16, 6, 64, 524288) < 16 * 524288 * 516


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def test_rejects_before_launch(L):
    import compressed_sparse_attention_csa2_amd as csa2
    n = None
    # compress: NULL kc
    s = L.csa2_compress(1, 4, FAKE, n, FAKE, FAKE, FAKE, FAKE, n, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                        FAKE, 8, 2, 0, n)
    assert s == 1 and b"NULL" in L.csa2_last_error()
    # compress: ratio 2 needs gate logits, ratio 1 does not; only ratios 1 and 2
    s = L.csa2_compress(1, 4, FAKE, FAKE, n, FAKE, FAKE, FAKE, n, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                        FAKE, 8, 2, 0, n)
    assert s == 1
    s = L.csa2_compress(1, 4, FAKE, FAKE, n, FAKE, FAKE, FAKE, n, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                        FAKE, 8, 3, 0, n)
    assert s == 3 and b"ratio" in L.csa2_last_error()
    # compress: negative T
    s = L.csa2_compress(1, -2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n, FAKE, FAKE, 16, FAKE, FAKE,
                        FAKE, FAKE, 8, 2, 0, n)
    assert s == 2
    # compress: neither projection nor given keys
    s = L.csa2_compress(1, 4, FAKE, FAKE, FAKE, FAKE, n, FAKE, n, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
                        FAKE, 8, 2, 0, n)
    assert s == 1
    # window: cap 0
    assert L.csa2_encode_window(1, 4, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 0, n) == 2
    # index: workspace too small
    s = L.csa2_index_topk(1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2, FAKE, FAKE, FAKE, 16, n)
    assert s == 5 and b"workspace" in L.csa2_last_error()
    s = L.csa2_index_topk(1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 0, FAKE, FAKE, FAKE, 16, n)
    assert s == 3 and b"ratio" in L.csa2_last_error()
    # attention: unsupported heads, small ring, missing workspace
    args = [FAKE] * 4 + [200, FAKE, FAKE, 64, 0] + [FAKE] * 5 + [16, FAKE, n, n, FAKE]
    assert L.csa2_sparse_attn(1, 8, 24, *args, 1 << 30, n) == 3
    args_ring = [FAKE] * 4 + [100, FAKE, FAKE, 64, 0] + [FAKE] * 5 + [16, FAKE, n, n, FAKE]
    assert L.csa2_sparse_attn(1, 8, 64, *args_ring, 1 << 30, n) == 4
    assert L.csa2_sparse_attn(4, 1, 64, *args, 0, n) == 5
    args_fmt = [FAKE] * 4 + [200, FAKE, FAKE, 64, 2] + [FAKE] * 5 + [16, FAKE, n, n, FAKE]
    assert L.csa2_sparse_attn(1, 8, 64, *args_fmt, 1 << 30, n) == 3
    # forward: decode without n_entries
    s = L.csa2_forward(1, 1, 64, FAKE, n, n, n, n, n, n, n, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                       FAKE, FAKE, FAKE, FAKE, 64, 2, 0, n, FAKE, FAKE, 128, FAKE, FAKE, FAKE, n,
                       n, FAKE, 1 << 30, n)
    assert s == 1 and b"n_entries" in L.csa2_last_error()
    # forward: ring smaller than T + 127
    s = L.csa2_forward(1, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, n, n, FAKE, FAKE, FAKE, FAKE, FAKE,
                       FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 32, 2, 0, n, FAKE, FAKE, 100, FAKE,
                       FAKE, FAKE, n, n, FAKE, 1 << 30, n)
    assert s == 4
    # encoders: bad widths
    assert L.csa2_encode_fp4_rows(FAKE, 4, 48, FAKE, FAKE, n) == 2
    assert L.csa2_encode_fp4e4_rows(FAKE, 4, 40, FAKE, FAKE, n) == 2
    assert L.csa2_decode_fp4e4_rows(FAKE, FAKE, 4, 24, FAKE, n) == 2
    assert L.csa2_encode_fp8_rows(FAKE, 4, 2048, FAKE, FAKE, n) == 2
    assert L.csa2_decode_fp8_rows(FAKE, 4, 12, FAKE, n) == 2
    # index-query quantiser: negative rows, NULL output
    assert L.csa2_quant_index_query(FAKE, FAKE, -1, FAKE, FAKE, n) == 2
    assert L.csa2_quant_index_query(FAKE, FAKE, 4, n, FAKE, n) == 1


def test_empty_calls_read_no_pointer(L):
    """T / Tq / rows = 0: CSA2_OK with every pointer NULL (nothing is launched)"""
    n = None
    assert L.csa2_compress(1, 0, n, n, n, n, n, n, n, n, n, 16, n, n, n, n, 8, 2, 0, n) == 0
    assert L.csa2_index_topk(1, 0, n, n, n, n, n, n, 64, 2, n, n, n, 0, n) == 0
    assert L.csa2_index_scores(1, 0, n, n, n, n, n, n, 64, 1, n, n, 0, n) == 0
    assert L.csa2_sparse_attn(1, 0, 64, n, n, n, n, 200, n, n, 64, 1, n, n, n, n, n, 16, n, n, n,
                              n, 0, n) == 0
    assert L.csa2_encode_fp4e4_rows(n, 0, 512, n, n, n) == 0
    assert L.csa2_quant_index_query(n, n, 0, n, n, n) == 0
    assert L.csa2_append(0, *([n] * 12), 16, n, n, n, n, 8, 2, 0, n, n, 128, n) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(csa2.CSA2Error, match="GPU"):
        csa2.csa2_encode_fp4_rows(x, torch.zeros(4, 16, dtype=torch.uint8),
                                  torch.zeros(4, 1, dtype=torch.uint8))


def test_product_path_has_no_oracle_import():
    """the library package never imports the oracle"""
    pkg = os.path.join(ROOT, "compressed_sparse_attention_csa2_amd")
    for dp, _, fs in os.walk(pkg):
        for f in fs:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dp, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "csa2_oracle" not in txt, f
