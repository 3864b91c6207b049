"""Oracle results for the synthetic workloads -- TEST INFRASTRUCTURE ONLY.

Builds the oracle's caches from the seeded inputs of ``csa2_synth`` and
evaluates selected query rows.  Used by the GPU parity tests, the smoke check
and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import time

import numpy as np

import csa2_synth as synth
from . import (compress, fp4_encode_rows_bf16, z_encode_rows_bf16, query_rows, window_encode,
               attend, TOPK, WINDOW)


class PrefillReference:
    """Oracle caches of one prefill workload (request b), then rows on demand."""

    def __init__(self, wl: synth.Workload, b: int = 0):
        assert wl.kind == "prefill"
        self.wl, self.b = wl, b
        T = wl.Tq
        self.cos, self.sin = synth.rope_table(wl.rope_rows)
        kc = wl.kc()[b:b + 1]
        gc = wl.gc()[b:b + 1] if wl.ratio == 2 else None     # ratio 1 reads no gates
        derive = wl.keys == "derive"
        ki_given = None if derive else wl.ki_given()[b:b + 1]
        self.z_codes, self.z_scales, self.ki_codes, self.ki_scales = compress(
            kc, gc, wl.gamma_c(), wl.w_ik() if derive else None, wl.gamma_ik(), ki_given,
            self.cos, self.sin, entry_stride=T // wl.ratio, ratio=wl.ratio, z_format=wl.z_format)
        self.n_entries = T // wl.ratio
        self.cap = wl.cap
        self.w_codes = np.zeros((1, wl.cap, 512), np.uint8)
        self.w_scale = np.zeros((1, wl.cap), np.float32)
        self._encoded = np.zeros(T, bool)
        self.wI = wl.wI()[b]
        self.sink = wl.sink()

    def window_full(self):
        wn = self.wl.wn()[self.b:self.b + 1]
        window_encode(wn, self.cos, self.sin, self.cap, 0, self.w_codes, self.w_scale)
        self._encoded[:] = True
        return self.w_codes[0], self.w_scale[0]

    def _ensure_window(self, rows):
        need = set()
        for t in rows:
            for p in range(max(0, t - (WINDOW - 1)), t + 1):
                if not self._encoded[p]:
                    need.add(p)
        for p in sorted(need):
            wn = self.wl.wn_rows(self.b, [p]).reshape(1, 1, 512)
            window_encode(wn, self.cos, self.sin, self.cap, p, self.w_codes, self.w_scale)
            self._encoded[p] = True

    def rows(self, t, want_scores=False, want_attn=True):
        t = np.asarray(t, np.int64)
        if want_attn:
            self._ensure_window(t)
        Q = self.wl.Q_rows(self.b, t) if want_attn else None
        return query_rows(t, self.n_entries, self.wl.qI_rows(self.b, t), self.wI[t], Q,
                          self.ki_codes[0], self.ki_scales[0], self.z_codes[0], self.z_scales[0],
                          self.w_codes[0], self.w_scale[0], self.cap, self.sink, self.cos,
                          self.sin, TOPK, want_scores=want_scores, ratio=self.wl.ratio,
                          z_format=self.wl.z_format)


class DecodeReference:
    """Oracle caches of one request of a decode workload, then its query rows."""

    def __init__(self, wl: synth.Workload, b: int):
        assert wl.kind == "decode"
        self.wl, self.b = wl, b
        N = wl.n_entries
        self.cos, self.sin = synth.rope_table(wl.rope_rows)
        chunk = 1 << 16
        self.ki_codes = np.zeros((N, 64), np.uint8)
        self.ki_scales = np.zeros((N, 4), np.uint8)
        for j0 in range(0, N, chunk):
            n = min(chunk, N - j0)
            cc, ss = fp4_encode_rows_bf16(wl.ki_rows(b, j0, n))
            self.ki_codes[j0:j0 + n] = cc
            self.ki_scales[j0:j0 + n] = ss
        wn = wl.wn()[b:b + 1]
        self.w_codes, self.w_scale = window_encode(wn, self.cos, self.sin, wl.cap, wl.win_pos0)
        self.w_codes, self.w_scale = self.w_codes[0], self.w_scale[0]
        self.sink = wl.sink()
        self.wI = wl.wI()[b]
        self.z_codes = np.zeros((N, 256), np.uint8)
        self.z_scales = np.zeros((N, 32 if wl.z_format == 1 else 16), np.uint8)
        self._z_done = np.zeros(N, bool)

    def _ensure_z(self, js):
        js = np.unique(js[js >= 0])
        js = js[~self._z_done[js]]
        if len(js) == 0:
            return
        rows = np.ascontiguousarray(self.b * self.wl.n_entries + js.astype(np.int64))
        raw = np.empty((len(js), 512), np.uint16)
        synth.lib().synth_normal_rows(self.wl.seed, synth.ID_ZROW, synth._ptr(rows), len(js),
                                      512, 1.0, 0.0, 1, synth._ptr(raw))
        cc, ss = z_encode_rows_bf16(raw, self.wl.z_format)
        self.z_codes[js] = cc
        self.z_scales[js] = ss
        self._z_done[js] = True

    def rows(self, qi, want_scores=False, want_attn=True):
        """qi: local query indices 0..Tq-1 of this request"""
        wl = self.wl
        qi = np.asarray(qi, np.int64)
        pos = wl.q_pos0 + qi
        qI = wl.qI()[self.b, qi]
        sel = query_rows(pos, wl.n_entries, qI, self.wI[qi], None, self.ki_codes, self.ki_scales,
                         None, None, None, None, wl.cap, self.sink, self.cos, self.sin, TOPK,
                         want_scores=want_scores, ratio=wl.ratio)
        if not want_attn:
            return sel
        self._ensure_z(sel["idx"].reshape(-1))
        Q = wl.Q()[self.b][:, qi, :].transpose(1, 0, 2)
        H = wl.H
        O = np.zeros((len(qi), H, 512))
        Ob = np.zeros((len(qi), H, 512), np.uint16)
        lse = np.zeros((len(qi), H))
        for i in range(len(qi)):
            O[i], lse[i], Ob[i] = attend(Q[i], int(pos[i]), self.w_codes, self.w_scale, wl.cap,
                                         self.z_codes, self.z_scales, sel["idx"][i],
                                         int(sel["cnt"][i]), self.sink, self.cos, self.sin,
                                         z_format=wl.z_format)
        sel.update(O=O, O_bf16=Ob, lse=lse)
        return sel


def time_oracle(fn, *a, **k):
    t0 = time.perf_counter()
    r = fn(*a, **k)
    return r, time.perf_counter() - t0
