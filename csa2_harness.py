"""GPU workload runner: seeded inputs -> device tensors -> CSA2 library calls.

Shared by the GPU tests, the smoke check and the benchmark.  It only moves the
seeded inputs of ``csa2_synth`` to the GPU, allocates outputs and workspace,
and calls the library through its Python binding; all computation happens in
the library's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

import compressed_sparse_attention_csa2_amd as csa2
import csa2_synth as synth

D, HI, DI, TOPK = 512, 32, 128, 512


def up(a: np.ndarray, dev="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def down(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


class PrefillRun:
    """B requests x T new tokens starting at position 0: compress, window, select, attend."""

    def __init__(self, wl: synth.Workload, dev="cuda"):
        assert wl.kind == "prefill"
        self.wl = wl
        B, T, H = wl.B, wl.Tq, wl.H
        self.stride = max(T // wl.ratio, 1)
        cos_t, sin_t = synth.rope_table(wl.rope_rows)
        self.rope_cos, self.rope_sin = up(cos_t, dev), up(sin_t, dev)
        self.kc, self.wn = up(wl.kc(), dev), up(wl.wn(), dev)
        self.gc = up(wl.gc(), dev) if wl.ratio == 2 else None     # ratio 1 reads no gates
        self.Q = up(wl.Q(), dev)
        self.qI, self.wI = up(wl.qI(), dev), up(wl.wI(), dev)
        self.gamma_c, self.gamma_ik = up(wl.gamma_c(), dev), up(wl.gamma_ik(), dev)
        derive = wl.keys == "derive"
        self.w_ik = up(wl.w_ik(), dev) if derive else None
        self.ki_given = None if derive else up(wl.ki_given(), dev)
        self.sink = up(wl.sink(), dev)
        self.pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
        u8 = torch.uint8
        self.z_codes = torch.zeros(B, self.stride, 256, dtype=u8, device=dev)
        zsb = 32 if wl.z_format == 1 else 16          # scale bytes per compressed row
        self.z_scales = torch.zeros(B, self.stride, zsb, dtype=u8, device=dev)
        self.ki_codes = torch.zeros(B, self.stride, 64, dtype=u8, device=dev)
        self.ki_scales = torch.zeros(B, self.stride, 4, dtype=u8, device=dev)
        self.w_codes = torch.zeros(B, wl.cap, D, dtype=u8, device=dev)
        self.w_scale = torch.zeros(B, wl.cap, dtype=torch.float32, device=dev)
        self.idx = torch.full((B, T, TOPK), -7, dtype=torch.int32, device=dev)
        self.cnt = torch.full((B, T), -7, dtype=torch.int32, device=dev)
        self.O = torch.zeros(B, H, T, D, dtype=torch.bfloat16, device=dev)
        self.lse = torch.zeros(B, H, T, dtype=torch.float32, device=dev)
        self.ws = csa2.workspace(csa2.OP_FORWARD, B, T, H, self.stride, dev)

    def forward(self, stream=None):
        csa2.csa2_forward(self.pos0, self.Q, self.qI, self.wI, self.sink, self.rope_cos,
                          self.rope_sin, self.z_codes, self.z_scales, self.ki_codes,
                          self.ki_scales, self.w_codes, self.w_scale, self.idx, self.cnt, self.O,
                          self.ws, kc=self.kc, gc=self.gc, wn=self.wn, gamma_c=self.gamma_c,
                          w_ik=self.w_ik, gamma_ik=self.gamma_ik, ki_given=self.ki_given,
                          lse=self.lse, stream=stream, ratio=self.wl.ratio,
                          z_format=self.wl.z_format)

    def fetch(self, big=True) -> dict:
        out = dict(z_codes=down(self.z_codes), z_scales=down(self.z_scales),
                   ki_codes=down(self.ki_codes), ki_scales=down(self.ki_scales),
                   w_codes=down(self.w_codes), w_scale=down(self.w_scale),
                   idx=down(self.idx), cnt=down(self.cnt))
        if big:
            out.update(O=down(self.O), lse=down(self.lse))
        return out


class DecodeRun:
    """B requests x Tq query tokens over caches filled from the seeded pre-quantisation rows."""

    def __init__(self, wl: synth.Workload, dev="cuda", chunk_rows: int = 1 << 16):
        assert wl.kind == "decode"
        self.wl = wl
        B, Tq, H, N = wl.B, wl.Tq, wl.H, wl.n_entries
        self.stride = N
        cos_t, sin_t = synth.rope_table(wl.rope_rows)
        self.rope_cos, self.rope_sin = up(cos_t, dev), up(sin_t, dev)
        u8 = torch.uint8
        self.z_codes = torch.zeros(B, N, 256, dtype=u8, device=dev)
        zsb = 32 if wl.z_format == 1 else 16          # scale bytes per compressed row
        self.z_scales = torch.zeros(B, N, zsb, dtype=u8, device=dev)
        enc_z = csa2.csa2_encode_fp4e4_rows if wl.z_format == 1 else csa2.csa2_encode_fp4_rows
        self.ki_codes = torch.zeros(B, N, 64, dtype=u8, device=dev)
        self.ki_scales = torch.zeros(B, N, 4, dtype=u8, device=dev)
        for b in range(B):
            for j0 in range(0, N, chunk_rows):
                n = min(chunk_rows, N - j0)
                z = up(wl.z_rows(b, j0, n), dev)
                enc_z(z, self.z_codes[b, j0:j0 + n].view(n, 256),
                      self.z_scales[b, j0:j0 + n].view(n, zsb))
                k = up(wl.ki_rows(b, j0, n), dev)
                csa2.csa2_encode_fp4_rows(k, self.ki_codes[b, j0:j0 + n].view(n, 64),
                                          self.ki_scales[b, j0:j0 + n].view(n, 4))
                del z, k
        self.w_codes = torch.zeros(B, wl.cap, D, dtype=u8, device=dev)
        self.w_scale = torch.zeros(B, wl.cap, dtype=torch.float32, device=dev)
        wpos = torch.full((B,), wl.win_pos0, dtype=torch.int32, device=dev)
        csa2.csa2_encode_window(wpos, up(wl.wn(), dev), self.rope_cos, self.rope_sin,
                                self.w_codes, self.w_scale)
        self.Q = up(wl.Q(), dev)
        self.qI, self.wI = up(wl.qI(), dev), up(wl.wI(), dev)
        self.sink = up(wl.sink(), dev)
        self.q_pos0 = torch.full((B,), wl.q_pos0, dtype=torch.int32, device=dev)
        self.n_entries = torch.full((B,), N, dtype=torch.int32, device=dev)
        self.idx = torch.full((B, Tq, TOPK), -7, dtype=torch.int32, device=dev)
        self.cnt = torch.full((B, Tq), -7, dtype=torch.int32, device=dev)
        self.O = torch.zeros(B, H, Tq, D, dtype=torch.bfloat16, device=dev)
        self.lse = torch.zeros(B, H, Tq, dtype=torch.float32, device=dev)
        self.ws = csa2.workspace(csa2.OP_FORWARD, B, Tq, H, N, dev)
        torch.cuda.synchronize()

    def forward(self, stream=None):
        csa2.csa2_forward(self.q_pos0, self.Q, self.qI, self.wI, self.sink, self.rope_cos,
                          self.rope_sin, self.z_codes, self.z_scales, self.ki_codes,
                          self.ki_scales, self.w_codes, self.w_scale, self.idx, self.cnt, self.O,
                          self.ws, n_entries=self.n_entries, lse=self.lse, stream=stream,
                          ratio=self.wl.ratio, z_format=self.wl.z_format)

    def fetch(self) -> dict:
        return dict(idx=down(self.idx), cnt=down(self.cnt), O=down(self.O), lse=down(self.lse))
