"""GPU parity of the decode append path (csa2_append) through the C ABI.

Appending tokens one at a time -- window row per token, the pair buffer held
between calls, an entry written when a pair closes -- must leave the same
cache bytes as compressing all tokens in one call, and the same bytes as the
oracle's compression of those tokens.  Requests start from prefills of
different lengths, one of them odd (its last token seeded into the pair
buffer), so every call mixes requests that open and close pairs.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def log(*a):
    print("[gpu]", *a, flush=True)


@pytest.mark.parametrize("zf", [0, 1])
@pytest.mark.parametrize("ratio", [2, 1])
@pytest.mark.parametrize("mode", ["derive", "given"])
def test_append_matches_prefill_and_oracle(mode, ratio, zf):
    """ratio 1: every appended token writes its own entry; no pair buffer, no gates.
    zf = 1: entries in the pages' per-16 E4M3 format"""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_csa2_amd as csa2
    import csa2_synth as synth
    import oracle
    from csa2_harness import up, down

    B, T, cap = 3, 40, 48
    stride = T // ratio + 4
    prefill = [10, 12, 11]
    seed = 0xC5A2A000
    kc = synth.normal(seed, 201, (B, T, 512))
    gc = synth.normal(seed, 202, (B, T, 512))
    wn = synth.normal(seed, 203, (B, T, 512))
    gamma_c = synth.normal(seed, 204, (512,), mul=0.1, add=1.0, dtype="f32")
    gamma_ik = synth.normal(seed, 206, (128,), mul=0.1, add=1.0, dtype="f32")
    if mode == "derive":
        w_ik = synth.normal(seed, 205, (512, 128), mul=1.0 / math.sqrt(512))
        ki = None
    else:
        w_ik = None
        ki = synth.normal(seed, 207, (B, T // ratio, 128))
    cos_t, sin_t = synth.rope_table(T)
    if ratio == 1:
        gc = None                           # never read at ratio 1
    log(f"csa2_append: mode={mode} ratio={ratio} B={B} T={T} prefill={prefill}")

    oz, ozs, ok_, oks = oracle.compress(kc, gc, gamma_c, w_ik, gamma_ik, ki, cos_t, sin_t, stride,
                                        ratio=ratio, z_format=zf)
    ow, ows = oracle.window_encode(wn, cos_t, sin_t, cap)

    def caches():
        return dict(z_codes=torch.zeros(B, stride, 256, dtype=torch.uint8, device="cuda"),
                    z_scales=torch.zeros(B, stride, 32 if zf else 16, dtype=torch.uint8,
                                         device="cuda"),
                    ki_codes=torch.zeros(B, stride, 64, dtype=torch.uint8, device="cuda"),
                    ki_scales=torch.zeros(B, stride, 4, dtype=torch.uint8, device="cuda"),
                    w_codes=torch.zeros(B, cap, 512, dtype=torch.uint8, device="cuda"),
                    w_scale=torch.zeros(B, cap, dtype=torch.float32, device="cuda"))

    g_gc, g_gik, g_cos, g_sin = up(gamma_c), up(gamma_ik), up(cos_t), up(sin_t)
    g_wik = None if w_ik is None else up(w_ik)
    g_kc, g_wn = up(kc), up(wn)
    g_gcl = None if gc is None else up(gc)

    # one call over all tokens
    A = caches()
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    csa2.csa2_compress(zero, g_kc, g_gcl, g_gc, g_wik, g_gik, None if ki is None else up(ki),
                       g_cos, g_sin, A["z_codes"], A["z_scales"], A["ki_codes"], A["ki_scales"],
                       ratio=ratio, z_format=zf)
    csa2.csa2_encode_window(zero, g_wn, g_cos, g_sin, A["w_codes"], A["w_scale"])

    # per-request prefills, then one token per call
    Bc = caches()
    pair_kc = torch.zeros(B, 512, dtype=torch.bfloat16, device="cuda") if ratio == 2 else None
    pair_gc = torch.zeros(B, 512, dtype=torch.bfloat16, device="cuda") if ratio == 2 else None
    z1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, P in enumerate(prefill):
        sl = {k: v[b:b + 1] for k, v in Bc.items()}
        csa2.csa2_compress(z1, up(kc[b:b + 1, :P]), None if gc is None else up(gc[b:b + 1, :P]),
                           g_gc, g_wik, g_gik,
                           None if ki is None else up(ki[b:b + 1, :P // ratio]), g_cos, g_sin,
                           sl["z_codes"], sl["z_scales"], sl["ki_codes"], sl["ki_scales"],
                           ratio=ratio, z_format=zf)
        csa2.csa2_encode_window(z1, up(wn[b:b + 1, :P]), g_cos, g_sin, sl["w_codes"], sl["w_scale"])
        if ratio == 2 and P % 2:
            pair_kc[b] = up(kc[b, P - 1])
            pair_gc[b] = up(gc[b, P - 1])
    for i in range(T - min(prefill)):
        pos = np.array([P + i if P + i < T else -1 for P in prefill], np.int32)
        take = np.maximum(pos, 0)
        ki_new = None
        if ki is not None:
            ki_new = up(np.ascontiguousarray(ki[np.arange(B), take // ratio]))
        csa2.csa2_append(up(pos), up(np.ascontiguousarray(kc[np.arange(B), take])),
                         None if gc is None else up(np.ascontiguousarray(gc[np.arange(B), take])),
                         up(np.ascontiguousarray(wn[np.arange(B), take])), pair_kc, pair_gc,
                         g_gc, g_wik, g_gik, ki_new, g_cos, g_sin, Bc["z_codes"], Bc["z_scales"],
                         Bc["ki_codes"], Bc["ki_scales"], Bc["w_codes"], Bc["w_scale"],
                         ratio=ratio, z_format=zf)
    torch.cuda.synchronize()

    n = T // ratio
    ref = dict(z_codes=oz, z_scales=ozs, ki_codes=ok_, ki_scales=oks, w_codes=ow, w_scale=ows)
    for k in ref:
        a, bb = down(A[k]), down(Bc[k])
        if k.startswith("w"):
            assert np.array_equal(bb, a), f"append vs one call: {k}"
            assert np.array_equal(bb, ref[k]), f"append vs oracle: {k}"
        else:
            assert np.array_equal(bb[:, :n], a[:, :n]), f"append vs one call: {k}"
            assert np.array_equal(bb[:, :n], ref[k][:, :n]), f"append vs oracle: {k}"
            assert not np.any(bb[:, n:]), f"rows past the last pair written: {k}"
    log("  append == one call == oracle (caches bit-exact)")
