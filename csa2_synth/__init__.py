"""Seeded synthetic inputs for the CSA2 attention layer (shared by the HIP tests and the oracle).

The module draws random numbers and shapes them into the workloads' input
distributions; it contains none of the attention method's arithmetic.  Every
tensor element is a pure function of (seed, tensor id, element index), so any
slice of any tensor can be regenerated on its own: the oracle recomputes just
the rows it checks, while the GPU side uploads whole tensors.

Workloads (shapes and distributions follow the five workload descriptions this
layer is measured on; what is not stated there is marked "recipe"):

* 0: prefill B=1, T=256, H=16; K^I derived from the compressed rows through a
  512x128 projection (recipe: W_IK ~ N(0,1)/sqrt(512), gain 1+0.1 N(0,1)).
* 1: prefill B=1, T=8192, H=64; K^I given, 64 Gaussian clusters
  (recipe: K^I_j = mu_c + 0.25 N(0, I), mu_c ~ N(0, I)).
* 2: prefill B=1, T=65536, H=64; as 1.
* 3: decode B=128 x 1 query at position 131071; 65536 entries per request;
  window ring of 128 slots; compressed rows and index keys N(0,1) (recipe).
* 4: verify-decode B=16 x 6 queries at positions 1048570..1048575; 524288
  entries; ring of 133 slots; K^I log-normal norms (sigma 1) with 1% exact
  duplicates of an earlier key; compressed rows N(0,1).

All activations are bf16 (stored as uint16), gains/weights of the indexer and
sinks are fp32.  The rotary table is an input too: cos/sin of p*theta^(-2i/64),
theta = 10000, computed in double and rounded once to fp32.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libcsa2synth.so")

# tensor ids
ID_KC, ID_GC, ID_WN, ID_Q, ID_QI, ID_WI = 1, 2, 3, 4, 5, 6
ID_GAMMA_C, ID_GAMMA_IK, ID_WIK, ID_SINK = 7, 8, 9, 10
ID_KI_NOISE, ID_KI_CENTRE, ID_KI_ASSIGN = 11, 12, 13
ID_ZROW, ID_KI_XI, ID_KI_G, ID_DUP_FLAG, ID_DUP_SRC = 14, 15, 16, 17, 18
ID_KI_FLAT = 19

D, ROPE_LO, WINDOW, HI, DI, TOPK = 512, 448, 128, 32, 128, 512
THETA = 10000.0


def build(verbose: bool = False) -> str:
    """Compile the generator library with gcc (OpenMP)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           os.path.join(_HERE, "synth.c"), "-o", _SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, u32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_void_p)
        L.synth_normal.argtypes = [u64, u32, i64, i64, dbl, dbl, ctypes.c_int, vp]
        L.synth_uniform.argtypes = [u64, u32, i64, i64, vp]
        L.synth_rope_table.argtypes = [dbl, i64, i64, ctypes.c_int, vp, vp]
        L.synth_clustered_rows.argtypes = [u64, u32, u32, u32, ctypes.c_int, dbl, i64, i64,
                                           ctypes.c_int, vp]
        L.synth_lognormal_rows.argtypes = [u64, u32, u32, u32, u32, dbl, dbl, i64, i64,
                                           ctypes.c_int, vp, vp]
        L.synth_normal_rows.argtypes = [u64, u32, vp, i64, ctypes.c_int, dbl, dbl, ctypes.c_int, vp]
        L.synth_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, tid: int, shape, mul=1.0, add=0.0, dtype="bf16", start: int = 0) -> np.ndarray:
    """add + mul * N(0,1), elements start .. start+prod(shape)-1 of tensor tid."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    lib().synth_normal(seed, tid, start, n, float(mul), float(add), 1 if dtype == "bf16" else 0,
                       _ptr(out))
    return out


def uniform(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform(seed, tid, start, n, _ptr(out))
    return out


def rope_table(rows: int, p0: int = 0, theta: float = THETA, pairs: int = 32):
    """cos, sin fp32 [rows, pairs] for absolute positions p0 .. p0+rows-1."""
    c = np.empty((rows, pairs), dtype=np.float32)
    s = np.empty((rows, pairs), dtype=np.float32)
    lib().synth_rope_table(float(theta), p0, rows, pairs, _ptr(c), _ptr(s))
    return c, s


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One workload's shapes and recipe.  Tensors are generated on demand."""
    cid: int
    kind: str            # "prefill" or "decode"
    B: int
    Tq: int              # query tokens per request
    H: int
    n_entries: int       # compressed entries per request after the call
    cap: int             # window ring capacity (slots)
    q_pos0: int          # absolute position of each request's first query token
    keys: str            # "derive" | "clustered" | "flat" | "lognormal_dup"
    seed: int = 0
    name: str = ""
    extra: dict = field(default_factory=dict)
    ratio: int = 2       # positions per compressed entry (2: pairs; 1: one entry per token)
    z_format: int = 0    # compressed-row storage: 0 one E8M0 scale per 32, 1 one E4M3 per 16

    # ---- geometry -------------------------------------------------------
    @property
    def rope_rows(self) -> int:
        return self.q_pos0 + self.Tq

    @property
    def win_pos0(self) -> int:
        """First absolute position held in the window ring."""
        return max(0, self.q_pos0 - (WINDOW - 1)) if self.kind == "decode" else self.q_pos0

    @property
    def win_rows(self) -> int:
        """Number of window rows written before attention (per request)."""
        return self.q_pos0 + self.Tq - self.win_pos0

    # ---- prefill tensors -----------------------------------------------
    def kc(self):
        return normal(self.seed, ID_KC, (self.B, self.Tq, D))

    def gc(self):
        return normal(self.seed, ID_GC, (self.B, self.Tq, D))

    def wn(self):
        """Window vectors for every position the ring receives, [B, win_rows, 512]."""
        return normal(self.seed, ID_WN, (self.B, self.win_rows, D))

    def wn_rows(self, b: int, pos) -> np.ndarray:
        """Window vectors of request b at absolute positions pos (in the ring)."""
        idx = np.ascontiguousarray(b * self.win_rows + (np.asarray(pos, np.int64) - self.win_pos0),
                                   dtype=np.int64)
        out = np.empty((len(idx), D), np.uint16)
        lib().synth_normal_rows(self.seed, ID_WN, _ptr(idx), len(idx), D,
                                1.0, 0.0, 1, _ptr(out))
        return out

    def Q(self):
        return normal(self.seed, ID_Q, (self.B, self.H, self.Tq, D))

    def Q_rows(self, b: int, t) -> np.ndarray:
        """Q[b, :, t, :] for local query indices t -> [len(t), H, 512]."""
        t = np.asarray(t, np.int64)
        rows = np.ascontiguousarray(
            ((b * self.H + np.arange(self.H)[None, :]) * self.Tq + t[:, None]).reshape(-1), np.int64)
        out = np.empty((len(t) * self.H, D), np.uint16)
        lib().synth_normal_rows(self.seed, ID_Q, _ptr(rows), len(rows), D,
                                1.0, 0.0, 1, _ptr(out))
        return out.reshape(len(t), self.H, D)

    def qI(self):
        return normal(self.seed, ID_QI, (self.B, self.Tq, HI, DI))

    def qI_rows(self, b: int, t) -> np.ndarray:
        t = np.asarray(t, np.int64)
        rows = np.ascontiguousarray(
            ((b * self.Tq + t[:, None]) * HI + np.arange(HI)[None, :]).reshape(-1), np.int64)
        out = np.empty((len(rows), DI), np.uint16)
        lib().synth_normal_rows(self.seed, ID_QI, _ptr(rows), len(rows), DI,
                                1.0, 0.0, 1, _ptr(out))
        return out.reshape(len(t), HI, DI)

    def wI(self):
        return normal(self.seed, ID_WI, (self.B, self.Tq, HI), mul=1.0 / 64.0, dtype="f32")

    def gamma_c(self):
        return normal(self.seed, ID_GAMMA_C, (D,), mul=0.1, add=1.0, dtype="f32")

    def gamma_ik(self):
        return normal(self.seed, ID_GAMMA_IK, (DI,), mul=0.1, add=1.0, dtype="f32")

    def w_ik(self):
        return normal(self.seed, ID_WIK, (D, DI), mul=1.0 / math.sqrt(D))

    def sink(self):
        return normal(self.seed, ID_SINK, (self.H,), dtype="f32")

    # ---- index keys (pre-quantisation values) ---------------------------
    def ki_rows(self, b: int, j0: int, n: int) -> np.ndarray:
        """Given-mode K^I rows j0 .. j0+n-1 of request b, bf16 [n, 128]."""
        out = np.empty((n, DI), np.uint16)
        jj = b * self.n_entries + j0
        if self.keys == "clustered":
            lib().synth_clustered_rows(self.seed, ID_KI_CENTRE, ID_KI_ASSIGN, ID_KI_NOISE, 64, 0.25,
                                       jj, n, DI, _ptr(out))
        elif self.keys == "flat":
            out = normal(self.seed, ID_KI_FLAT, (n, DI), start=jj * DI)
        elif self.keys == "lognormal_dup":
            # duplicates point at earlier keys of the same request
            root = np.empty(n, np.int64)
            tmp = np.empty((n, DI), np.uint16)
            lib().synth_lognormal_rows(self.seed + 7919 * (b + 1), ID_KI_XI, ID_KI_G, ID_DUP_FLAG,
                                       ID_DUP_SRC, 1.0, 0.01, j0, n, DI, _ptr(tmp), _ptr(root))
            out = tmp
        else:
            raise ValueError("derive-mode workloads have no given keys")
        return out

    def ki_given(self):
        n = self.Tq // self.ratio if self.kind == "prefill" else self.n_entries
        return np.stack([self.ki_rows(b, 0, n) for b in range(self.B)])

    def z_rows(self, b: int, j0: int, n: int) -> np.ndarray:
        """Decode-cache compressed rows (pre-quantisation), bf16 [n, 512]."""
        return normal(self.seed, ID_ZROW, (n, D), start=(b * self.n_entries + j0) * D)


def workload(cid: int, T: int | None = None, H: int | None = None, ratio: int = 2,
             z_format: int = 0) -> Workload:
    """The five measured workloads; T/H overrides give same-recipe smaller prefills, ratio 1
    the one-entry-per-token form of a prefill."""
    seed = 0xC5A20000 + cid
    tag = ("" if ratio == 2 else f" ratio {ratio}") + ("" if z_format == 0 else " Z per-16 E4M3")
    if cid == 0:
        T = T or 256
        return Workload(cid, "prefill", 1, T, H or 16, T // ratio, T + WINDOW - 1, 0, "derive",
                        seed, f"prefill T={T} H={H or 16} derived index keys{tag}", ratio=ratio,
                        z_format=z_format)
    if cid in (1, 2):
        T = T or (8192 if cid == 1 else 65536)
        return Workload(cid, "prefill", 1, T, H or 64, T // ratio, T + WINDOW - 1, 0, "clustered",
                        seed, f"prefill T={T} H={H or 64} clustered index keys{tag}", ratio=ratio,
                        z_format=z_format)
    if cid == 3:
        return Workload(3, "decode", 128, 1, H or 64, 65536, 128, 131071, "flat", seed,
                        "decode B=128 x 1 @ 131072 context")
    if cid == 4:
        return Workload(4, "decode", 16, 6, H or 64, 524288, 133, 1048570, "lognormal_dup", seed,
                        "verify-decode B=16 x 6 @ 1048576 context")
    raise ValueError(cid)


def decode_workload(B: int, Tq: int, n_entries: int, H: int = 64, keys: str = "flat",
                    seed: int = 0xC5A20010, q_pos0: int | None = None,
                    ratio: int = 2, z_format: int = 0) -> Workload:
    """A decode workload with the recipe of workloads 3/4 (ratio 2), or its one-entry-per-token
    form (ratio 1): the queries follow the last entry's positions."""
    q0 = (ratio * n_entries - Tq) if q_pos0 is None else q_pos0
    tag = ("" if ratio == 2 else f" ratio {ratio}") + ("" if z_format == 0 else " Z per-16 E4M3")
    return Workload(99, "decode", B, Tq, H, n_entries, Tq + WINDOW - 1, q0, keys, seed,
                    f"decode B={B} x {Tq} @ {ratio * n_entries}{tag}", ratio=ratio,
                    z_format=z_format)
