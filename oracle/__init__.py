"""CSA2 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Python marshalling around the plain C oracle in ``csa2_oracle.c``.  Only the
test-suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP library never does, and this package never imports the
HIP library.  Inputs come from ``csa2_synth`` (seeded, shared by both sides);
no input or expected value here is ever produced by the GPU path.

Parity status of each function (what pins it) is listed in the tests under
``tests/test_oracle_*.py``.  The one part with no independent pin is the
end-to-end value of the attention output on random inputs: beyond the
identities those tests check (sink identity against a library SDPA, the t=0
closed form, MQA symmetry, the value bound), its parity is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_ORACLE_LIB names another build of the oracle to load (the tests' sanitizer build)
_SO = os.environ.get("CSA2_ORACLE_LIB") or os.path.join(_HERE, "libcsa2oracle.so")

D, ROPE_LO, WINDOW, HI, DI, TOPK = 512, 448, 128, 32, 128, 512
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, os.path.join(_HERE, "csa2_oracle.c"), "-o", _SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def build_sanitized(out: str, cc: str = "/opt/rocm/llvm/bin/clang") -> str:
    """the oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (clang, so that
    it shares one sanitizer runtime with the host-sanitized HIP library)"""
    cmd = [cc, *CFLAGS, "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", os.path.join(_HERE, "csa2_oracle.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            if os.environ.get("CSA2_ORACLE_LIB"):
                raise FileNotFoundError(_SO)
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_e2m1_value.argtypes = [i32]
        L.orc_e2m1_value.restype = f32
        L.orc_e2m1_encode.argtypes = [f32]
        L.orc_e4m3_value.argtypes = [i32]
        L.orc_e4m3_value.restype = f32
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_exp.argtypes = [f32]
        L.orc_exp.restype = f32
        L.orc_fp4_encode.argtypes = [vp, i32, vp, vp]
        L.orc_fp4_value.argtypes = [vp, vp, i32]
        L.orc_fp4_value.restype = ctypes.c_double
        L.orc_fp8_encode_row.argtypes = [vp, i32, vp, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i32, vp]
        L.orc_compress_entry.argtypes = [vp] * 16 + [i32]
        L.orc_compress.argtypes = [i32, i32, i32] + [vp] * 12 + [i64, i32, i32]
        L.orc_fp4e4_encode.argtypes = [vp, i32, vp, vp]
        L.orc_fp4e4_value.argtypes = [vp, vp, i32]
        L.orc_fp4e4_value.restype = ctypes.c_double
        L.orc_fp4e4_encode_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_window_encode.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp]
        L.orc_fp4_encode_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_fp8_encode_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_index_scores.argtypes = [vp, vp, vp, vp, vp, i64, vp]
        L.orc_topk.argtypes = [vp, i64, i32, vp]
        L.orc_topk.restype = i32
        L.orc_quant_index_query.argtypes = [vp, vp, vp]
        L.orc_attend.argtypes = [vp, i32, i64, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i64,
                                 i32]
        L.orc_query_rows.argtypes = [i32, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32,
                                     vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, i32]
        _lib = L
    return _lib


class _Args:
    """Pointer marshalling that keeps every converted array alive until the
    owning function returns (a temporary's address must not outlive it)."""

    def __init__(self):
        self.keep = []

    def __call__(self, a, dt=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt) if dt is not None else a
        assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous numpy"
        self.keep.append(a)
        return a.ctypes.data


def c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode(y: float) -> int:
    return lib().orc_e2m1_encode(y)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(y)


def fp4_encode(x: np.ndarray):
    """x [rows, n] fp32 -> codes [rows, n/2] u8, scales [rows, n/32] u8"""
    A = _Args()
    x = c(x, np.float32)
    rows, n = x.shape
    codes = np.zeros((rows, n // 2), np.uint8)
    scales = np.zeros((rows, n // 32), np.uint8)
    for r in range(rows):
        lib().orc_fp4_encode(A(x[r]), n, A(codes[r]), A(scales[r]))
    return codes, scales


def fp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """exact values (double) of FP4 rows"""
    A = _Args()
    codes = c(codes, np.uint8)
    scales = c(scales, np.uint8)
    rows = codes.shape[0]
    n = codes.shape[1] * 2
    out = np.empty((rows, n), np.float64)
    for r in range(rows):
        for k in range(n):
            out[r, k] = lib().orc_fp4_value(A(codes[r]), A(scales[r]), k)
    return out


def fp4e4_encode(x: np.ndarray):
    """the pages' format: x [rows, n] fp32 -> codes [rows, n/2] u8, E4M3 scales [rows, n/16] u8"""
    A = _Args()
    x = c(x, np.float32)
    rows, n = x.shape
    codes = np.zeros((rows, n // 2), np.uint8)
    scales = np.zeros((rows, n // 16), np.uint8)
    for r in range(rows):
        lib().orc_fp4e4_encode(A(x[r]), n, A(codes[r]), A(scales[r]))
    return codes, scales


def fp4e4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """exact values (double) of rows in the pages' format"""
    A = _Args()
    codes = c(codes, np.uint8)
    scales = c(scales, np.uint8)
    rows = codes.shape[0]
    n = codes.shape[1] * 2
    out = np.empty((rows, n), np.float64)
    for r in range(rows):
        pc, ps = A(codes[r]), A(scales[r])
        for k in range(n):
            out[r, k] = lib().orc_fp4e4_value(pc, ps, k)
    return out


def fp4e4_encode_rows_bf16(x: np.ndarray):
    A = _Args()
    x = c(x, np.uint16)
    rows, n = x.shape
    codes = np.zeros((rows, n // 2), np.uint8)
    scales = np.zeros((rows, n // 16), np.uint8)
    lib().orc_fp4e4_encode_rows(A(x), rows, n, A(codes), A(scales))
    return codes, scales


def z_encode_rows_bf16(x: np.ndarray, z_format: int = 0):
    """Z rows in storage format z_format (0: one E8M0 scale per 32; 1: one E4M3 per 16)"""
    return fp4e4_encode_rows_bf16(x) if z_format == 1 else fp4_encode_rows_bf16(x)


def fp8_encode_row(x: np.ndarray):
    A = _Args()
    x = c(x, np.float32)
    codes = np.zeros(x.shape[0], np.uint8)
    s = np.zeros(1, np.float32)
    lib().orc_fp8_encode_row(A(x), x.shape[0], A(codes), A(s))
    return codes, float(s[0])


def fp4_encode_rows_bf16(x: np.ndarray):
    A = _Args()
    x = c(x, np.uint16)
    rows, n = x.shape
    codes = np.zeros((rows, n // 2), np.uint8)
    scales = np.zeros((rows, n // 32), np.uint8)
    lib().orc_fp4_encode_rows(A(x), rows, n, A(codes), A(scales))
    return codes, scales


def fp8_encode_rows_bf16(x: np.ndarray):
    A = _Args()
    x = c(x, np.uint16)
    rows, n = x.shape
    codes = np.zeros((rows, n), np.uint8)
    sc = np.zeros(rows, np.float32)
    lib().orc_fp8_encode_rows(A(x), rows, n, A(codes), A(sc))
    return codes, sc


def exp32(x: float) -> float:
    return lib().orc_exp(x)


def rmsnorm(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    A = _Args()
    x = c(x, np.float32)
    g = c(gamma, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(A(x), A(g), x.shape[0], A(y))
    return y


# ---------------------------------------------------------------- steps
def compress_entry(kc0, kc1, gc0, gc1, gamma_c, w_ik, gamma_ik, ki_given, cs, sn, z_format=0):
    """one entry; returns (z_codes, z_scales, ki_codes, ki_scales, z_pre, ki_pre).
    kc1 = None: compression ratio one, the entry is the one position kc0 (gates unused).
    z_format 1: Z in the pages' format (32 E4M3 scale bytes)."""
    A = _Args()
    zc = np.zeros(256, np.uint8)
    zs = np.zeros(32 if z_format == 1 else 16, np.uint8)
    kc_ = np.zeros(64, np.uint8)
    ks = np.zeros(4, np.uint8)
    zp = np.zeros(512, np.float32)
    kp = np.zeros(128, np.float32)
    args = [c(kc0, np.uint16), c(kc1, np.uint16), c(gc0, np.uint16), c(gc1, np.uint16),
            c(gamma_c, np.float32), None if w_ik is None else c(w_ik, np.uint16),
            c(gamma_ik, np.float32), None if ki_given is None else c(ki_given, np.uint16),
            c(cs, np.float32), c(sn, np.float32)]
    lib().orc_compress_entry(*[A(a) for a in args], A(zc), A(zs), A(kc_), A(ks), A(zp), A(kp),
                             z_format)
    return zc, zs, kc_, ks, zp, kp


def compress(kc, gc, gamma_c, w_ik, gamma_ik, ki_given, cos_t, sin_t, entry_stride, pos0=0,
             ratio=2, z_format=0):
    """kc, gc [B,T,512] bf16 -> caches [B, entry_stride, ...]: entries pos0/2 .. (pos0+T)/2-1
    pooled from pairs (ratio 2), or entries pos0 .. pos0+T-1, one per position, rotated at
    their own position (ratio 1, "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV
    Cache", CSA2 section; gc may be None)."""
    assert ratio in (1, 2)
    A = _Args()
    kc = c(kc, np.uint16)
    gc = c(gc, np.uint16)
    B, T, _ = kc.shape
    z_codes = np.zeros((B, entry_stride, 256), np.uint8)
    z_scales = np.zeros((B, entry_stride, 32 if z_format == 1 else 16), np.uint8)
    ki_codes = np.zeros((B, entry_stride, 64), np.uint8)
    ki_scales = np.zeros((B, entry_stride, 4), np.uint8)
    lib().orc_compress(B, T, pos0, A(kc), A(gc), A(gamma_c, np.float32),
                       A(None if w_ik is None else c(w_ik, np.uint16)), A(gamma_ik, np.float32),
                       A(None if ki_given is None else c(ki_given, np.uint16)),
                       A(cos_t, np.float32), A(sin_t, np.float32),
                       A(z_codes), A(z_scales), A(ki_codes), A(ki_scales), entry_stride, ratio,
                       z_format)
    return z_codes, z_scales, ki_codes, ki_scales


def window_encode(wn, cos_t, sin_t, cap, pos0=0, w_codes=None, w_scale=None):
    """wn [B,T,512] bf16 at positions pos0.. -> ring [B,cap,512] codes, [B,cap] scales"""
    A = _Args()
    wn = c(wn, np.uint16)
    B, T, _ = wn.shape
    if w_codes is None:
        w_codes = np.zeros((B, cap, 512), np.uint8)
        w_scale = np.zeros((B, cap), np.float32)
    lib().orc_window_encode(B, T, pos0, A(wn), A(cos_t, np.float32), A(sin_t, np.float32),
                            cap, A(w_codes), A(w_scale))
    return w_codes, w_scale


def quant_index_query(q):
    A = _Args()
    q = c(q, np.uint16)
    q8 = np.zeros((32, 128), np.uint8)
    sq = np.zeros(32, np.float32)
    lib().orc_quant_index_query(A(q), A(q8), A(sq))
    return q8, sq


def index_scores(q8, sq, w, ki_codes, ki_scales, n):
    A = _Args()
    S = np.zeros(max(n, 1), np.float32)
    lib().orc_index_scores(A(q8, np.uint8), A(sq, np.float32), A(w, np.float32),
                           A(ki_codes, np.uint8), A(ki_scales, np.uint8), n, A(S))
    return S[:n]


def topk(S, n, k=TOPK):
    A = _Args()
    idx = np.zeros(k, np.int32)
    cnt = lib().orc_topk(A(S, np.float32), n, k, A(idx))
    return idx, cnt



# Hierarchical candidate pool ("Inside DeepSeek V4.1", the Hierarchical Sparse
# Indexer paragraph; "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV
# Cache", section "Hierarchical indexing bounds the later searches"): blocks of
# 8 entries, 2,048 blocks (16,384 candidates) kept, the newest block always.
POOL_BLOCK, POOL_BLOCKS = 8, 2048


def pool_blocks(S, n, block=POOL_BLOCK, keep=POOL_BLOCKS):
    """Blocks of the candidate pool, ascending.  Entries 0..n-1 are cut into
    blocks of `block` (the last one may be short); a block's key is the largest
    index score in it.  The pool holds the block with the newest entry (n-1)
    and, of the other blocks, the keep-1 with the largest keys (ties: the
    smaller block) -- every block when there are at most `keep`."""
    S = np.asarray(S, np.float32)
    nb = (n + block - 1) // block
    if nb <= keep:
        return np.arange(nb, dtype=np.int32)
    keys = [float(S[b * block:min(n, (b + 1) * block)].max()) for b in range(nb - 1)]
    ranked = sorted(range(nb - 1), key=lambda b: (-keys[b], b))
    return np.array(sorted(ranked[:keep - 1]) + [nb - 1], np.int32)


def pool_entries(pool, n, block=POOL_BLOCK):
    """Entries of the pool's blocks below n, ascending."""
    if len(pool) == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(b * block, min(n, (b + 1) * block), dtype=np.int64)
                           for b in pool])


def reindex_topk(q8, sq, w, ki_codes, ki_scales, n, pool, block=POOL_BLOCK, k=TOPK):
    """Reindex selection: the layer's own index query scores only the pool's
    candidates against the shared index keys and keeps the top k of them with
    the rule of topk (score desc, entry asc), in ascending order, -1 padded.
    Returns (idx, cnt, candidates, their scores)."""
    cand = pool_entries(pool, n, block)
    Sc = index_scores(q8, sq, w, np.ascontiguousarray(ki_codes[cand]),
                      np.ascontiguousarray(ki_scales[cand]), len(cand))
    pos, cnt = topk(Sc, len(cand), k)
    idx = np.full(k, -1, np.int32)
    idx[:cnt] = cand[pos[:cnt]]
    return idx, cnt, cand, Sc

def attend(Q, p, w_codes, w_scale, cap, z_codes, z_scales, idx, cnt, sink, cos_t, sin_t,
           w_floor=0, z_format=0):
    """Q [H,512] bf16 -> O [H,512] double, lse [H], O_bf16 [H,512].  w_floor: the
    start s of a bounded replay ("Inside DeepSeek V4.1 Flash: Deriving the 890-Byte
    KV Cache", section "Bounded replay trades exact state for cheaper
    resumption"): the window is max(s, p-127) .. p."""
    A = _Args()
    Q = c(Q, np.uint16)
    H = Q.shape[0]
    O = np.zeros((H, 512), np.float64)
    lse = np.zeros(H, np.float64)
    Ob = np.zeros((H, 512), np.uint16)
    lib().orc_attend(A(Q), H, p, A(w_codes, np.uint8), A(w_scale, np.float32), cap,
                     A(z_codes, np.uint8), A(z_scales, np.uint8), A(idx, np.int32), cnt,
                     A(sink, np.float32), A(cos_t, np.float32), A(sin_t, np.float32),
                     A(O), A(lse), A(Ob), int(w_floor), int(z_format))
    return O, lse, Ob


def query_rows(pos, n_entries, qI, wI, Q, ki_codes, ki_scales, z_codes, z_scales, w_codes,
               w_scale, cap, sink, cos_t, sin_t, k=TOPK, want_scores=False, want_O=True,
               ratio=2, z_format=0):
    """Selection and attention for query tokens of ONE request (caches of that request).
    A query at p sees entries j < min(floor((p+1)/ratio), n_entries)."""
    A = _Args()
    pos = c(pos, np.int64)
    nq = pos.shape[0]
    H = Q.shape[1] if Q is not None else 0
    idx = np.zeros((nq, k), np.int32)
    cnt = np.zeros(nq, np.int32)
    O = np.zeros((nq, H, 512), np.float64) if (Q is not None and want_O) else None
    Ob = np.zeros((nq, H, 512), np.uint16) if Q is not None else None
    lse = np.zeros((nq, H), np.float64) if Q is not None else None
    S = np.zeros((nq, max(n_entries, 1)), np.float32) if want_scores else None
    lib().orc_query_rows(nq, A(pos), n_entries, A(qI, np.uint16), A(wI, np.float32),
                         A(None if Q is None else c(Q, np.uint16)), H,
                         A(ki_codes, np.uint8), A(ki_scales, np.uint8),
                         A(z_codes, np.uint8), A(z_scales, np.uint8),
                         A(w_codes, np.uint8), A(w_scale, np.float32), cap,
                         A(sink, np.float32), A(cos_t, np.float32), A(sin_t, np.float32),
                         k, A(idx), A(cnt), A(O), A(Ob), A(lse), A(S), ratio, z_format)
    return dict(idx=idx, cnt=cnt, O=O, O_bf16=Ob, lse=lse, S=S)
