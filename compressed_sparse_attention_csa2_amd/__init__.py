"""CSA2 attention layer for MI355X: Python binding of libcsa2.so.

Argument marshalling only: every function here checks tensor dtypes/devices,
passes raw device pointers and the current HIP stream to the C ABI of the same
name (include/csa2.h) and raises on a non-OK status.  All computation happens
in the library's HIP kernels; there is no fallback path.  PyTorch provides
device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIB names another build of the same library to load (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("CSA2_LIB") or os.path.join(_HERE, "libcsa2.so")

D, WINDOW, HI, DI, TOPK = 512, 128, 32, 128, 512
OP_INDEX_TOPK, OP_SPARSE_ATTN, OP_FORWARD, OP_INDEX_SCORES, OP_INDEX_POOL, OP_REINDEX = 1, 2, 3, 4, 5, 6
POOL_BLOCKS = 2048
ABI_VERSION = 3

_lib = None


class CSA2Error(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CSA2Error(f"{LIB_PATH} is missing: build it first (python -c "
                            "'import __graft_entry__; __graft_entry__.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.csa2_abi_version.restype = i32
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_status_string.argtypes = [i32]
        L.csa2_workspace_size.restype = sz
        L.csa2_workspace_size.argtypes = [i32, i32, i32, i32, i64]
        L.csa2_compress.argtypes = [i32, i32] + [vp] * 9 + [i64] + [vp] * 4 + [i64, i32, i32, vp]
        L.csa2_encode_window.argtypes = [i32, i32, vp, vp, vp, vp, i64, vp, vp, i32, vp]
        L.csa2_append.argtypes = [i32] + [vp] * 12 + [i64] + [vp] * 4 + [i64, i32, i32, vp, vp,
                                                                          i32, vp]
        L.csa2_index_topk.argtypes = [i32, i32] + [vp] * 6 + [i64, i32, vp, vp, vp, sz, vp]
        L.csa2_index_scores.argtypes = [i32, i32] + [vp] * 6 + [i64, i32, vp, vp, sz, vp]
        L.csa2_index_pool.argtypes = [i32, i32] + [vp] * 6 + [i64, i32] + [vp] * 5 + [sz, vp]
        L.csa2_reindex_topk.argtypes = [i32, i32] + [vp] * 6 + [i64, i32] + [vp] * 5 + [sz, vp]
        L.csa2_sparse_attn.argtypes = ([i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, i64, i32] +
                                       [vp] * 5 + [i64, vp, vp, vp, vp, sz, vp])
        L.csa2_forward.argtypes = ([i32, i32, i32] + [vp] * 14 + [i64] + [vp] * 4 + [i64, i32, i32,
                                   vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp])
        L.csa2_quant_index_query.argtypes = [vp, vp, i64, vp, vp, vp]
        L.csa2_index_topk_noalloc.argtypes = [i32, i32] + [vp] * 6 + [i64, i32, vp, vp, vp]
        L.csa2_encode_fp4_rows.argtypes = [vp, i64, i32, vp, vp, vp]
        L.csa2_encode_fp8_rows.argtypes = [vp, i64, i32, vp, vp, vp]
        L.csa2_decode_fp4_rows.argtypes = [vp, vp, i64, i32, vp, vp]
        L.csa2_encode_fp4e4_rows.argtypes = [vp, i64, i32, vp, vp, vp]
        L.csa2_decode_fp4e4_rows.argtypes = [vp, vp, i64, i32, vp, vp]
        L.csa2_decode_fp8_rows.argtypes = [vp, i64, i32, vp, vp]
        for name in ("csa2_compress", "csa2_encode_window", "csa2_append", "csa2_index_topk",
                     "csa2_index_scores", "csa2_index_pool", "csa2_reindex_topk", "csa2_sparse_attn",
                     "csa2_forward", "csa2_encode_fp4_rows", "csa2_encode_fp8_rows",
                     "csa2_decode_fp4_rows", "csa2_decode_fp8_rows", "csa2_encode_fp4e4_rows",
                     "csa2_decode_fp4e4_rows", "csa2_quant_index_query",
                     "csa2_index_topk_noalloc"):
            getattr(L, name).restype = i32
        if L.csa2_abi_version() != ABI_VERSION:
            raise CSA2Error("libcsa2.so ABI version mismatch")
        _lib = L
    return _lib


def _check(status: int, name: str):
    if status != 0:
        msg = lib().csa2_last_error().decode()
        kind = lib().csa2_status_string(status).decode()
        raise CSA2Error(f"{name}: {kind} ({status}): {msg}")


_DT = {"bf16": torch.uint16, "u8": torch.uint8, "f32": torch.float32, "i32": torch.int32}


def _p(t, dt=None, name="tensor"):
    """device pointer of a contiguous CUDA tensor (None -> NULL)"""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise CSA2Error(f"{name}: must live on the GPU")
    if not t.is_contiguous():
        raise CSA2Error(f"{name}: must be contiguous")
    if dt is not None:
        want = _DT[dt]
        ok = t.dtype == want or (dt == "bf16" and t.dtype == torch.bfloat16)
        if not ok:
            raise CSA2Error(f"{name}: dtype {t.dtype}, expected {dt}")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(op: int, B: int, Tq: int, H: int, entry_stride: int) -> int:
    return int(lib().csa2_workspace_size(op, B, Tq, H, entry_stride))


def workspace(op: int, B: int, Tq: int, H: int, entry_stride: int, device="cuda") -> torch.Tensor:
    n = workspace_size(op, B, Tq, H, entry_stride)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def csa2_compress(pos0, kc, gc, gamma_c, w_ik, gamma_ik, ki_given, rope_cos, rope_sin, z_codes,
                  z_scales, ki_codes, ki_scales, stream=None, ratio=2, z_format=0):
    B, T = kc.shape[0], kc.shape[1]
    _check(lib().csa2_compress(B, T, _p(pos0, "i32", "pos0"), _p(kc, "bf16", "kc"),
                               _p(gc, "bf16", "gc"), _p(gamma_c, "f32", "gamma_c"),
                               _p(w_ik, "bf16", "w_ik"), _p(gamma_ik, "f32", "gamma_ik"),
                               _p(ki_given, "bf16", "ki_given"), _p(rope_cos, "f32", "rope_cos"),
                               _p(rope_sin, "f32", "rope_sin"), rope_cos.shape[0],
                               _p(z_codes, "u8", "z_codes"), _p(z_scales, "u8", "z_scales"),
                               _p(ki_codes, "u8", "ki_codes"), _p(ki_scales, "u8", "ki_scales"),
                               z_codes.shape[1], ratio, z_format, _stream(stream)),
           "csa2_compress")


def csa2_encode_window(pos0, wn, rope_cos, rope_sin, w_codes, w_scale, stream=None):
    B, T = wn.shape[0], wn.shape[1]
    _check(lib().csa2_encode_window(B, T, _p(pos0, "i32", "pos0"), _p(wn, "bf16", "wn"),
                                    _p(rope_cos, "f32", "rope_cos"), _p(rope_sin, "f32", "rope_sin"),
                                    rope_cos.shape[0], _p(w_codes, "u8", "w_codes"),
                                    _p(w_scale, "f32", "w_scale"), w_codes.shape[1],
                                    _stream(stream)), "csa2_encode_window")



def csa2_append(pos, kc, gc, wn, pair_kc, pair_gc, gamma_c, w_ik, gamma_ik, ki_given, rope_cos,
                rope_sin, z_codes, z_scales, ki_codes, ki_scales, w_codes, w_scale, stream=None,
                ratio=2, z_format=0):
    B = kc.shape[0]
    _check(lib().csa2_append(B, _p(pos, "i32", "pos"), _p(kc, "bf16", "kc"), _p(gc, "bf16", "gc"),
                             _p(wn, "bf16", "wn"), _p(pair_kc, "bf16", "pair_kc"),
                             _p(pair_gc, "bf16", "pair_gc"), _p(gamma_c, "f32", "gamma_c"),
                             _p(w_ik, "bf16", "w_ik"), _p(gamma_ik, "f32", "gamma_ik"),
                             _p(ki_given, "bf16", "ki_given"), _p(rope_cos, "f32", "rope_cos"),
                             _p(rope_sin, "f32", "rope_sin"), rope_cos.shape[0],
                             _p(z_codes, "u8", "z_codes"), _p(z_scales, "u8", "z_scales"),
                             _p(ki_codes, "u8", "ki_codes"), _p(ki_scales, "u8", "ki_scales"),
                             z_codes.shape[1], ratio, z_format, _p(w_codes, "u8", "w_codes"),
                             _p(w_scale, "f32", "w_scale"), w_codes.shape[1], _stream(stream)),
           "csa2_append")

def csa2_index_topk(q_pos0, n_entries, qI, wI, ki_codes, ki_scales, idx, cnt, ws, stream=None,
                    ratio=2):
    B, Tq = qI.shape[0], qI.shape[1]
    _check(lib().csa2_index_topk(B, Tq, _p(q_pos0, "i32", "q_pos0"),
                                 _p(n_entries, "i32", "n_entries"), _p(qI, "bf16", "qI"),
                                 _p(wI, "f32", "wI"), _p(ki_codes, "u8", "ki_codes"),
                                 _p(ki_scales, "u8", "ki_scales"), ki_codes.shape[1], ratio,
                                 _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"), _p(ws, None, "ws"),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "csa2_index_topk")



NOALLOC_SCRATCH_BYTES = 64 << 20


def csa2_index_topk_noalloc(q_pos0, n_entries, qI, wI, ki_codes, ki_scales, idx, cnt,
                            stream=None, ratio=2):
    """csa2_index_topk with the library's own scratch array (no workspace argument)"""
    B, Tq = qI.shape[0], qI.shape[1]
    _check(lib().csa2_index_topk_noalloc(B, Tq, _p(q_pos0, "i32", "q_pos0"),
                                         _p(n_entries, "i32", "n_entries"), _p(qI, "bf16", "qI"),
                                         _p(wI, "f32", "wI"), _p(ki_codes, "u8", "ki_codes"),
                                         _p(ki_scales, "u8", "ki_scales"), ki_codes.shape[1],
                                         ratio, _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"),
                                         _stream(stream)),
           "csa2_index_topk_noalloc")


def csa2_index_pool(q_pos0, n_entries, qI, wI, ki_codes, ki_scales, idx, cnt, pool, pool_cnt, ws,
                    stream=None, ratio=2):
    B, Tq = qI.shape[0], qI.shape[1]
    _check(lib().csa2_index_pool(B, Tq, _p(q_pos0, "i32", "q_pos0"),
                                 _p(n_entries, "i32", "n_entries"), _p(qI, "bf16", "qI"),
                                 _p(wI, "f32", "wI"), _p(ki_codes, "u8", "ki_codes"),
                                 _p(ki_scales, "u8", "ki_scales"), ki_codes.shape[1], ratio,
                                 _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"),
                                 _p(pool, "i32", "pool"), _p(pool_cnt, "i32", "pool_cnt"),
                                 _p(ws, None, "ws"), ws.numel() * ws.element_size(),
                                 _stream(stream)),
           "csa2_index_pool")


def csa2_reindex_topk(q_pos0, n_entries, qI, wI, ki_codes, ki_scales, pool, pool_cnt, idx, cnt,
                      ws, stream=None, ratio=2):
    B, Tq = qI.shape[0], qI.shape[1]
    _check(lib().csa2_reindex_topk(B, Tq, _p(q_pos0, "i32", "q_pos0"),
                                   _p(n_entries, "i32", "n_entries"), _p(qI, "bf16", "qI"),
                                   _p(wI, "f32", "wI"), _p(ki_codes, "u8", "ki_codes"),
                                   _p(ki_scales, "u8", "ki_scales"), ki_codes.shape[1], ratio,
                                   _p(pool, "i32", "pool"), _p(pool_cnt, "i32", "pool_cnt"),
                                   _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"),
                                   _p(ws, None, "ws"), ws.numel() * ws.element_size(),
                                   _stream(stream)),
           "csa2_reindex_topk")

def csa2_index_scores(q_pos0, n_entries, qI, wI, ki_codes, ki_scales, scores, ws, stream=None,
                      ratio=2):
    B, Tq = qI.shape[0], qI.shape[1]
    _check(lib().csa2_index_scores(B, Tq, _p(q_pos0, "i32", "q_pos0"),
                                   _p(n_entries, "i32", "n_entries"), _p(qI, "bf16", "qI"),
                                   _p(wI, "f32", "wI"), _p(ki_codes, "u8", "ki_codes"),
                                   _p(ki_scales, "u8", "ki_scales"), ki_codes.shape[1], ratio,
                                   _p(scores, "f32", "scores"), _p(ws, None, "ws"),
                                   ws.numel() * ws.element_size(), _stream(stream)),
           "csa2_index_scores")


def csa2_sparse_attn(q_pos0, Q, w_codes, w_scale, z_codes, z_scales, idx, cnt, sink, rope_cos,
                     rope_sin, O, lse, ws, stream=None, win_floor=None, z_format=0):
    B, H, Tq = Q.shape[0], Q.shape[1], Q.shape[2]
    _check(lib().csa2_sparse_attn(B, Tq, H, _p(q_pos0, "i32", "q_pos0"), _p(Q, "bf16", "Q"),
                                  _p(w_codes, "u8", "w_codes"), _p(w_scale, "f32", "w_scale"),
                                  w_codes.shape[1], _p(z_codes, "u8", "z_codes"),
                                  _p(z_scales, "u8", "z_scales"), z_codes.shape[1], z_format,
                                  _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"),
                                  _p(sink, "f32", "sink"), _p(rope_cos, "f32", "rope_cos"),
                                  _p(rope_sin, "f32", "rope_sin"), rope_cos.shape[0],
                                  _p(O, "bf16", "O"), _p(lse, "f32", "lse"),
                                  _p(win_floor, "i32", "win_floor"), _p(ws, None, "ws"),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "csa2_sparse_attn")


def csa2_forward(pos0, Q, qI, wI, sink, rope_cos, rope_sin, z_codes, z_scales, ki_codes,
                 ki_scales, w_codes, w_scale, idx, cnt, O, ws, kc=None, gc=None, wn=None,
                 gamma_c=None, w_ik=None, gamma_ik=None, ki_given=None, n_entries=None, lse=None,
                 stream=None, ratio=2, z_format=0, win_floor=None):
    B, H, T = Q.shape[0], Q.shape[1], Q.shape[2]
    _check(lib().csa2_forward(B, T, H, _p(pos0, "i32", "pos0"), _p(kc, "bf16", "kc"),
                              _p(gc, "bf16", "gc"), _p(wn, "bf16", "wn"),
                              _p(gamma_c, "f32", "gamma_c"), _p(w_ik, "bf16", "w_ik"),
                              _p(gamma_ik, "f32", "gamma_ik"), _p(ki_given, "bf16", "ki_given"),
                              _p(Q, "bf16", "Q"), _p(qI, "bf16", "qI"), _p(wI, "f32", "wI"),
                              _p(sink, "f32", "sink"), _p(rope_cos, "f32", "rope_cos"),
                              _p(rope_sin, "f32", "rope_sin"), rope_cos.shape[0],
                              _p(z_codes, "u8", "z_codes"), _p(z_scales, "u8", "z_scales"),
                              _p(ki_codes, "u8", "ki_codes"), _p(ki_scales, "u8", "ki_scales"),
                              z_codes.shape[1], ratio, z_format, _p(n_entries, "i32", "n_entries"),
                              _p(w_codes, "u8", "w_codes"), _p(w_scale, "f32", "w_scale"),
                              w_codes.shape[1], _p(idx, "i32", "idx"), _p(cnt, "i32", "cnt"),
                              _p(O, "bf16", "O"), _p(lse, "f32", "lse"),
                              _p(win_floor, "i32", "win_floor"), _p(ws, None, "ws"),
                              ws.numel() * ws.element_size(), _stream(stream)), "csa2_forward")


def csa2_quant_index_query(qI, wI, q8, wq, stream=None):
    """qI [..., 128] bf16 and wI [...] fp32 with the same leading shape -> q8 codes, wq"""
    rows = wI.numel()
    if qI.numel() != rows * DI or q8.numel() != rows * DI or wq.numel() != rows:
        raise CSA2Error("csa2_quant_index_query: qI/q8 need 128 values per wI element")
    _check(lib().csa2_quant_index_query(_p(qI, "bf16", "qI"), _p(wI, "f32", "wI"), rows,
                                        _p(q8, "u8", "q8"), _p(wq, "f32", "wq"), _stream(stream)),
           "csa2_quant_index_query")


def csa2_encode_fp4_rows(x, codes, scales, stream=None):
    rows, cols = x.shape
    _check(lib().csa2_encode_fp4_rows(_p(x, "bf16", "x"), rows, cols, _p(codes, "u8", "codes"),
                                      _p(scales, "u8", "scales"), _stream(stream)),
           "csa2_encode_fp4_rows")


def csa2_encode_fp8_rows(x, codes, scale, stream=None):
    rows, cols = x.shape
    _check(lib().csa2_encode_fp8_rows(_p(x, "bf16", "x"), rows, cols, _p(codes, "u8", "codes"),
                                      _p(scale, "f32", "scale"), _stream(stream)),
           "csa2_encode_fp8_rows")


def csa2_decode_fp4_rows(codes, scales, out, stream=None):
    rows, cols = out.shape
    _check(lib().csa2_decode_fp4_rows(_p(codes, "u8", "codes"), _p(scales, "u8", "scales"), rows,
                                      cols, _p(out, "bf16", "out"), _stream(stream)),
           "csa2_decode_fp4_rows")


def csa2_encode_fp4e4_rows(x, codes, scales, stream=None):
    rows, cols = x.shape
    _check(lib().csa2_encode_fp4e4_rows(_p(x, "bf16", "x"), rows, cols, _p(codes, "u8", "codes"),
                                        _p(scales, "u8", "scales"), _stream(stream)),
           "csa2_encode_fp4e4_rows")


def csa2_decode_fp4e4_rows(codes, scales, out, stream=None):
    rows, cols = out.shape
    _check(lib().csa2_decode_fp4e4_rows(_p(codes, "u8", "codes"), _p(scales, "u8", "scales"),
                                        rows, cols, _p(out, "bf16", "out"), _stream(stream)),
           "csa2_decode_fp4e4_rows")


def csa2_decode_fp8_rows(codes, out, stream=None):
    rows, cols = out.shape
    _check(lib().csa2_decode_fp8_rows(_p(codes, "u8", "codes"), rows, cols,
                                      _p(out, "bf16", "out"), _stream(stream)),
           "csa2_decode_fp8_rows")
