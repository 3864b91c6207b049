"""Benchmark of the CSA2 attention layer on one MI355X.

A step is one csa2_forward over one batch of synthetic inputs: compression of
the new positions, window rows, lightning indexer + top-512, and the sparse
attention.  Default workload: prefill B=1, T=65536, 64 heads (32768
compressed entries).  A second object reports the batched decode workload
(128 requests x 1 query at 131072 context).  Inputs are seeded synthetic
tensors already resident in device memory when timing starts.

Prints ONE JSON line.  Roofline figures use algorithmic work only:
  indexer scores  8192 FLOP per (query, candidate entry) pair (32 heads x 128 x 2)
  attention       4 * 512 * H FLOP per (query, attended row) (QK^T and PV)
  decode bytes    68 B per scanned index key + gathered rows + Q/O/window
and are divided by the kernel's average duration measured here with HIP
events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8 = 5.0e15       # dense FP8 MFMA, FLOP/s
PEAK_BF16 = 2.5e15      # dense BF16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # HBM3E, B/s

# HBM bytes per launch counted by rocprofv3 (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, factors from
# a 1 GiB device copy; profiles/hbm_traffic_prefill_T65536_decode_B128.txt).  A figure is valid only
# for the kernel sources it was taken on: reported as null once any listed file has changed.
TRAFFIC = {
    ("k_attn", "prefill", 65536): (2.0005e+10, {
        "attention.hip": "96b2726c8cfc0b9d54466acc24f2ec26fce49ee6639160644ca9c27364a87401",
        "csa2_device.h": "134fb61f73efbe5f457591414f833043a952f213f0ef3fd121a73d33f90c0881"}),
    ("k_index_select", "prefill", 65536): (4.8043e+08, {
        "index_select.hip": "379c201f58b7c75543d72111b0d9cfffd73f736db9747b93b3ccad3f49bf4ca7",
        "index_device.h": "0acd7979927cedfd769d0d2bc055ab7118f0556847fcd84d3738b3b2a3260522",
        "csa2_device.h": "134fb61f73efbe5f457591414f833043a952f213f0ef3fd121a73d33f90c0881"}),
    ("k_fs_scan", "decode", 131072): (5.8564e+08, {
        "decode_select.hip": "c540a14f8813d7e03290fe744d3637f0e16f4c3a89a7ae114331a0357ee79d74",
        "index_device.h": "0acd7979927cedfd769d0d2bc055ab7118f0556847fcd84d3738b3b2a3260522",
        "csa2_device.h": "134fb61f73efbe5f457591414f833043a952f213f0ef3fd121a73d33f90c0881"}),
}


def measured_traffic(kernel: str, mode: str, size: int):
    """counter-measured HBM bytes per launch, or None if not measured on the current sources"""
    import hashlib
    ent = TRAFFIC.get((kernel, mode, size))
    if ent is None:
        return None
    csrc = os.path.join(ROOT, "compressed_sparse_attention_csa2_amd", "csrc")
    for name, digest in ent[1].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return ent[0]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def prefill_work(T: int, H: int):
    """algorithmic FLOPs of the indexer scores and of attention for a T-token prefill"""
    idx_pairs = sum((t + 1) // 2 for t in range(T))
    rows = sum(min(t + 1, 128) + min((t + 1) // 2, 512) for t in range(T))
    return 8192.0 * idx_pairs, 4.0 * 512 * H * rows


def decode_bytes(B: int, Tq: int, N: int, H: int) -> float:
    """minimum HBM bytes of one decode step (per request: the index-key scan,
    gathered compressed rows, window rows, queries, outputs, indexer queries)"""
    per_req = (68.0 * N + Tq * 512 * 272 + (127 + Tq) * 516 + Tq * (2 * H * 512 * 2)
               + Tq * (32 * 128 * 2 + 32 * 4))
    return B * per_req


def time_events(fn, steps: int, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / steps      # ms per call


def stage_times(run, steps: int, stream):
    """per-stage ms (each stage is one ABI call) measured with events on the launch stream"""
    import torch
    import compressed_sparse_attention_csa2_amd as csa2
    ws_i = run.ws
    r = run.wl.ratio
    out = {}
    if hasattr(run, "kc"):
        out["compress"] = time_events(lambda: csa2.csa2_compress(
            run.pos0, run.kc, run.gc, run.gamma_c, run.w_ik, run.gamma_ik, run.ki_given,
            run.rope_cos, run.rope_sin, run.z_codes, run.z_scales, run.ki_codes, run.ki_scales,
            ratio=r, z_format=run.wl.z_format), steps, stream)
        out["window"] = time_events(lambda: csa2.csa2_encode_window(
            run.pos0, run.wn, run.rope_cos, run.rope_sin, run.w_codes, run.w_scale), steps, stream)
        q_pos0 = run.pos0
        n_ent = torch.full_like(run.pos0, run.stride)
    else:
        q_pos0, n_ent = run.q_pos0, run.n_entries
    scores = torch.empty(run.idx.shape[0], run.idx.shape[1], run.stride, dtype=torch.float32,
                         device="cuda")
    out["index_scores"] = time_events(lambda: csa2.csa2_index_scores(
        q_pos0, n_ent, run.qI, run.wI, run.ki_codes, run.ki_scales, scores, ws_i, ratio=r), steps,
        stream)
    del scores
    out["index_topk"] = time_events(lambda: csa2.csa2_index_topk(
        q_pos0, n_ent, run.qI, run.wI, run.ki_codes, run.ki_scales, run.idx, run.cnt, ws_i,
        ratio=r), steps, stream)
    out["sparse_attn"] = time_events(lambda: csa2.csa2_sparse_attn(
        q_pos0, run.Q, run.w_codes, run.w_scale, run.z_codes, run.z_scales, run.idx, run.cnt,
        run.sink, run.rope_cos, run.rope_sin, run.O, run.lse, run.ws, z_format=run.wl.z_format),
        steps, stream)
    return out


def host_cpu():
    """host CPU model and the cores this process may use"""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def cpu_baseline_prefill(wl, n_rows: int):
    """the oracle on a bounded sample: all compression + n_rows query rows spread
    over T, once on one thread (Oracle-1) and once on all usable cores (Oracle-N:
    the same single-threaded routine on disjoint rows; the C oracle releases the
    interpreter lock inside each call and keeps no shared state)"""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle.reference import PrefillReference
    model, nproc, usable = host_cpu()
    t0 = time.perf_counter()
    ref = PrefillReference(wl)
    t_compress = time.perf_counter() - t0
    ref.window_full()
    rows = np.linspace(0, wl.Tq - 1, n_rows).astype(np.int64)
    t1 = time.perf_counter()
    for t in rows:
        ref.rows([t])
    t_rows = time.perf_counter() - t1
    per_token_1 = t_compress / wl.Tq + t_rows / n_rows
    nthr = max(1, min(16, usable))
    # Oracle-N: compression in nthr chunks of positions, then the rows, each on
    # nthr threads (every call its own outputs)
    import oracle
    import csa2_synth as synth
    derive = wl.keys == "derive"
    kc, gc = wl.kc(), (wl.gc() if wl.ratio == 2 else None)
    kig = None if derive else wl.ki_given()
    cos_t, sin_t = synth.rope_table(wl.rope_rows)
    step = -(-wl.Tq // nthr // 2) * 2
    spans = [(p, min(wl.Tq, p + step)) for p in range(0, wl.Tq, step)]
    r = wl.ratio

    def comp(span):
        p0, p1 = span
        oracle.compress(kc[:, p0:p1], None if gc is None else gc[:, p0:p1], wl.gamma_c(),
                        wl.w_ik() if derive else None, wl.gamma_ik(),
                        None if kig is None else kig[:, p0 // r:p1 // r], cos_t, sin_t,
                        entry_stride=wl.Tq // r, pos0=p0, ratio=r, z_format=wl.z_format)
    t2 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(comp, spans))
    t_compress_n = time.perf_counter() - t2
    t3 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(lambda t: ref.rows([t]), rows))
    t_rows_n = time.perf_counter() - t3
    per_token_n = t_compress_n / wl.Tq + t_rows_n / n_rows
    return {"value": 1.0 / per_token_n, "unit": "query-tokens/s", "cores": nthr, "kind": "oracle",
            "sample": f"full compression of {wl.Tq} positions + {n_rows} query rows evenly spaced "
                      f"over t=0..{wl.Tq - 1}; the single-threaded C oracle on {nthr} threads "
                      f"over disjoint position chunks ({t_compress_n:.2f} s) and rows "
                      f"({t_rows_n:.2f} s); rate = 1 / (compress s/token + row s/row), the rows' "
                      "mean time standing for all 65,536 rows",
            "host_cpu": model, "nproc": nproc, "usable_cores": usable,
            "oracle_1": {"value": 1.0 / per_token_1, "unit": "query-tokens/s", "cores": 1,
                         "seconds": {"compress": t_compress, "rows": t_rows}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=65536, help="prefill length (default: 65536)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "pool", "decode1", "decode1z", "pool1",
                                       "copy", "read", "verify", "prefill8k"], default=None,
                    help="time a single workload (for profiling runs); 'copy' runs a plain "
                         "1 GiB device copy, the calibration kernel for the HBM byte counters; "
                         "decode1 / pool1 are the ratio-1 forms, decode1z the ratio-1 form with "
                         "the pages' 288-byte rows; 'read' a read-only streaming kernel over 2 GiB "
                         "(the ceiling a scan can reach); verify / prefill8k the verify-decode and "
                         "8,192-token prefill workloads alone")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU; sharding it across GPUs is not "
                                   "implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import csa2_harness
    import csa2_synth as synth
    import compressed_sparse_attention_csa2_amd as csa2
    csa2.lib()
    assert torch.cuda.is_available(), "bench needs a GPU"
    stream = torch.cuda.current_stream()

    result = {}
    if args.only == "copy":
        n = 1 << 30
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.warmup, 1)):
            dst.copy_(src)
        ms = time_events(lambda: dst.copy_(src), args.steps, stream)
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                          "GB/s": 2 * n / (ms * 1e-3) / 1e9}), flush=True)
        return
    if args.only == "read":
        result["read"] = read_ceiling(args, stream)
        print(json.dumps(result), flush=True)
        return
    if args.only in ("verify", "prefill8k"):
        (run_verify if args.only == "verify" else run_prefill_small)(args, result, stream)
        print(json.dumps(result), flush=True)
        return
    wl = synth.workload(2, T=args.T) if args.T != 8192 else synth.workload(1)
    if args.only in ("decode", "pool", "decode1", "pool1", "decode1z"):
        args.no_cpu = True
        if args.only.startswith("decode"):
            run_decode(args, result, stream, ratio=1 if "1" in args.only else 2,
                       z_format=1 if args.only.endswith("z") else 0)
        else:
            run_pool(args, result, stream, ratio=1 if args.only.endswith("1") else 2)
        print(json.dumps(result), flush=True)
        return
    # ---------------------------------------------------------------- prefill
    log(f"generating inputs: {wl.name}")
    t0 = time.time()
    run = csa2_harness.PrefillRun(wl)
    torch.cuda.synchronize()
    log(f"inputs resident ({time.time() - t0:.1f} s); warmup {args.warmup}")
    for _ in range(args.warmup):
        run.forward()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_start = time.perf_counter()
    ms = time_events(run.forward, args.steps, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) / args.steps * 1e3
    log(f"prefill: {ms:.3f} ms/step (wall {wall:.3f})")
    stages = stage_times(run, args.steps, stream)
    log(f"stages (ms): {json.dumps({k: round(v, 4) for k, v in stages.items()})}")
    flop_idx, flop_att = prefill_work(wl.Tq, wl.H)
    t_att = stages["sparse_attn"] * 1e-3
    t_sel = stages["index_topk"] * 1e-3
    att = {"kernel": "k_attn (gather, QK on the stored rows, sink softmax, bf16 PV, inverse "
                     "rotation; csa2_sparse_attn also runs k_z_fp8_rows first, ~0.02 ms of the "
                     "timed call, which re-encodes the FP4 compressed rows as E4M3)",
           "bound": "mfma", "achieved": flop_att / t_att / 1e12, "peak": PEAK_BF16 / 1e12,
           "unit": "TFLOP/s", "flop_per_launch": flop_att,
           "traffic": measured_traffic("k_attn", "prefill", wl.Tq)}
    sel = {"kernel": "k_index_select (csa2_index_topk: the q^I E4M3 pass, then scores and the "
                     "streaming top-512 in one kernel; no score row in memory)",
           "bound": "mfma", "achieved": flop_idx / t_sel / 1e12, "peak": PEAK_FP8 / 1e12,
           "unit": "TFLOP/s", "flop_per_launch": flop_idx,
           "traffic": measured_traffic("k_index_select", "prefill", wl.Tq)}
    for d in (att, sel):
        d["frac"] = d["achieved"] / d["peak"]
    dom, other = (att, sel) if t_att >= t_sel else (sel, att)
    value = wl.Tq / (ms * 1e-3)
    mixed_time = flop_idx / PEAK_FP8 + flop_att / PEAK_BF16
    result.update({
        "metric": "CSA2 query-tokens/s (prefill T=64K; decode B=128@128K) + % of MFMA/HBM roofline",
        "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "indexer: fp8 (E4M3 query) x fp4 (E2M1 key) MFMA; attention: QK as a two-term "
                 "E4M3 query on the scaled fp8/fp4 MFMA against the stored rows, PV bf16 MFMA; "
                 "fp32 accumulation and softmax",
        "data": "synthetic (seeded; shapes and distributions of the workload description)",
        "config": {"workload": f"CSA2 prefill B=1 T={wl.Tq} H={wl.H} d=512 window 128 "
                               f"top-512, {wl.Tq // 2} compressed entries, clustered index keys",
                   "global_batch": 1, "seq_len": wl.Tq, "parallelism": "none (1 GPU)"},
        "roofline": dom,
        "roofline_other": other,
        "stages_ms": stages,
        "mixed_roofline_frac": mixed_time / (ms * 1e-3),
        "fp8_peak_frac_literal": (flop_idx + flop_att) / (ms * 1e-3) / PEAK_FP8,
    })
    del run
    torch.cuda.empty_cache()
    if args.only is None and args.T == 65536:
        run_prefill_small(args, result, stream)
    if not args.no_decode and args.only is None:
        result["read_ceiling"] = read_ceiling(args, stream)
        run_decode(args, result, stream)
        run_verify(args, result, stream)
        run_pool(args, result, stream)
        run_decode(args, result, stream, ratio=1)
        run_decode(args, result, stream, ratio=1, z_format=1)
        run_pool(args, result, stream, ratio=1)

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu:
        log(f"timing the CPU oracle on {args.cpu_rows} rows")
        result["cpu_baseline"] = cpu_baseline_prefill(wl, args.cpu_rows)
    print(json.dumps(result), flush=True)


def read_ceiling(args, stream):
    """HBM read bandwidth of a plain streaming read over 2 GiB (libcsa2calib.so)"""
    import ctypes
    import torch
    from compressed_sparse_attention_csa2_amd import _build
    if not os.path.exists(_build.CALIB):
        raise RuntimeError(f"{_build.CALIB} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(_build.CALIB)
    L.csa2_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    n = 2 << 30
    buf = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    best = None
    for blocks in (2048, 4096, 8192):
        f = lambda: L.csa2_calib_read(buf.data_ptr(), n, sink.data_ptr(), blocks, sp)
        assert f() == 0
        ms = time_events(f, max(args.steps, 10), stream)
        gbs = n / (ms * 1e-3) / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": gbs, "bytes": n, "ms": ms, "blocks": blocks}
    del buf
    torch.cuda.empty_cache()
    best["frac_of_8TBps"] = best["GB/s"] * 1e9 / PEAK_HBM
    log(f"read ceiling: {best['GB/s']:.0f} GB/s ({best['blocks']} blocks)")
    return best


def run_prefill_small(args, result, stream):
    """The 8,192-token prefill (workload 1) as one csa2_forward per step."""
    import torch
    import csa2_harness
    import csa2_synth as synth
    wl = synth.workload(1)
    log(f"generating inputs: {wl.name}")
    run = csa2_harness.PrefillRun(wl)
    for _ in range(args.warmup):
        run.forward()
    torch.cuda.synchronize()
    ms = time_events(run.forward, args.steps, stream)
    st = stage_times(run, args.steps, stream)
    flop_idx, flop_att = prefill_work(wl.Tq, wl.H)
    mixed = flop_idx / PEAK_FP8 + flop_att / PEAK_BF16
    log(f"prefill T={wl.Tq}: {ms:.3f} ms/step; stages {json.dumps({k: round(v, 4) for k, v in st.items()})}")
    result["prefill_T8192"] = {
        "workload": f"CSA2 prefill B=1 T={wl.Tq} H={wl.H}, {wl.Tq // 2} compressed entries, "
                    "clustered index keys",
        "value": wl.Tq / (ms * 1e-3), "unit": "query-tokens/s", "ms_per_step": ms,
        "stages_ms": st, "mixed_roofline_frac": mixed / (ms * 1e-3),
        "attention_bf16_frac": flop_att / (st["sparse_attn"] * 1e-3) / PEAK_BF16}
    del run
    torch.cuda.empty_cache()


def run_verify(args, result, stream):
    """The speculative-verify decode (workload 4: B=16 x 6 queries over 524,288 entries)
    as one csa2_forward per step; near the ridge, so both fractions are given: the
    step's time at the MFMA peaks (FP8 indexer + BF16 attention) and at the HBM peak
    (index-key scan + gathered rows + Q/O + window), each over the measured time."""
    import torch
    import csa2_harness
    import csa2_synth as synth
    wl = synth.workload(4)
    log(f"generating caches: {wl.name}")
    t0 = time.time()
    run = csa2_harness.DecodeRun(wl)
    log(f"caches resident ({time.time() - t0:.1f} s)")
    for _ in range(args.warmup):
        run.forward()
    torch.cuda.synchronize()
    ms = time_events(run.forward, args.steps, stream)
    st = stage_times(run, args.steps, stream)
    rows = wl.B * wl.Tq
    pairs = wl.B * sum(min((wl.q_pos0 + t + 1) // 2, wl.n_entries) for t in range(wl.Tq))
    flop_idx = 8192.0 * pairs
    flop_att = 4.0 * 512 * wl.H * rows * 640
    t_mfma = flop_idx / PEAK_FP8 + flop_att / PEAK_BF16
    nbytes = decode_bytes(wl.B, wl.Tq, wl.n_entries, wl.H)
    log(f"verify decode: {ms:.4f} ms/step; stages {json.dumps({k: round(v, 4) for k, v in st.items()})}")
    result["verify_decode"] = {
        "workload": "CSA2 speculative-verify decode B=16 x 6 queries at 1048570..1048575, "
                    "524,288 FP4 entries per request (log-normal key norms, 1% exact duplicates), "
                    "window 133, H=64, top-512",
        "value": rows / (ms * 1e-3), "unit": "query-tokens/s", "ms_per_step": ms,
        "stages_ms": st, "flop": {"indexer_fp8": flop_idx, "attention": flop_att},
        "mfma_roofline_frac": t_mfma / (ms * 1e-3), "hbm_bytes": nbytes,
        "hbm_roofline_frac": nbytes / (ms * 1e-3) / PEAK_HBM}
    del run
    torch.cuda.empty_cache()


def run_decode(args, result, stream, ratio=2, z_format=0):
    """Batched decode B=128 x 1 query at position 131071.  ratio 2: the measured
    workload (65,536 pooled entries per request); ratio 1: its decoder-layer form
    (131,072 entries, one per position); z_format 1: compressed rows in the pages'
    288-byte format (one E4M3 scale per 16), attended by the dequantising kernel."""
    import dataclasses
    import torch
    import csa2_harness
    import csa2_synth as synth
    if True:
        dwl = synth.workload(3)
        if ratio == 1:
            dwl = dataclasses.replace(dwl, n_entries=dwl.q_pos0 + 1, ratio=1,
                                      name=dwl.name + " ratio 1")
        if z_format == 1:
            dwl = dataclasses.replace(dwl, z_format=1, name=dwl.name + " Z per-16 E4M3")
        key = ("decode" if ratio == 2 else "decode_ratio1") + ("_z16" if z_format == 1 else "")
        log(f"generating caches: {dwl.name}")
        t0 = time.time()
        drun = csa2_harness.DecodeRun(dwl)
        log(f"caches resident ({time.time() - t0:.1f} s)")
        for _ in range(args.warmup):
            drun.forward()
        torch.cuda.synchronize()
        dms = time_events(drun.forward, args.steps, stream)
        dstages = stage_times(drun, args.steps, stream)
        log(f"{key}: {dms:.4f} ms/step; stages {json.dumps({k: round(v, 4) for k, v in dstages.items()})}")
        nbytes = decode_bytes(dwl.B, dwl.Tq, dwl.n_entries, dwl.H)
        scan_bytes = 68.0 * dwl.n_entries * dwl.B
        result[key] = {
            "workload": f"CSA2 batched decode B=128 x 1 query, 131072 context ({dwl.n_entries} "
                        f"FP4 entries at compression ratio {ratio}, "
                        f"{'288-byte (E4M3 per 16)' if z_format else '272-byte (E8M0 per 32)'} "
                        "rows, + 128 FP8 window rows), H=64, top-512",
            "value": dwl.B * dwl.Tq / (dms * 1e-3), "unit": "query-tokens/s", "ms_per_step": dms,
            "stages_ms": dstages,
            "hbm_frac_step": nbytes / (dms * 1e-3) / PEAK_HBM,
            # the selection stage (csa2_index_topk): threshold from a sample, the
            # index-key scan keeping only candidates, the cut; its bytes are the scan's
            "roofline": {"kernel": "k_fs_threshold + k_fs_scan + k_fs_select (index-key scan "
                                   "with the top-512 cut; no score rows)", "bound": "hbm",
                         "achieved": scan_bytes / (dstages["index_topk"] * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": scan_bytes / (dstages["index_topk"] * 1e-3) / PEAK_HBM,
                         "bytes_per_launch": scan_bytes,
                         "traffic": measured_traffic("k_fs_scan", "decode",
                                                     dwl.q_pos0 + 1) if ratio == 2 else None},
        }
        if "read_ceiling" in result:
            rc = result["read_ceiling"]["GB/s"] * 1e9
            result[key]["roofline"]["frac_of_read_ceiling"] = (
                scan_bytes / (dstages["index_topk"] * 1e-3) / rc)
            result[key]["hbm_frac_step_of_read_ceiling"] = nbytes / (dms * 1e-3) / rc
        # attention's own traffic: the selected rows, the window rows, Q and O
        zrow = 288.0 if z_format else 272.0
        att_bytes = dwl.B * dwl.Tq * (512 * zrow + 128 * 516 + 2 * dwl.H * 512 * 2)
        result[key]["attention"] = {
            "kernel": "k_attn_dq (dequantise to bf16 in LDS, bf16 MFMA)" if z_format else
                      "k_attn (FP8/FP4 scaled MFMA QK, bf16 MFMA PV)",
            "ms": dstages["sparse_attn"], "bytes": att_bytes,
            "GB/s": att_bytes / (dstages["sparse_attn"] * 1e-3) / 1e9,
            "frac_hbm": att_bytes / (dstages["sparse_attn"] * 1e-3) / PEAK_HBM}
        # decode append (one new token per request, half of them closing a pair):
        # window row, pair buffer, entry of a completed pair, into the same caches
        import compressed_sparse_attention_csa2_amd as csa2
        B = dwl.B
        gen = torch.Generator(device="cuda").manual_seed(5)
        rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=gen).to(torch.bfloat16)
        a_kc, a_gc, a_wn, a_ki = rnd(B, 512), rnd(B, 512), rnd(B, 512), rnd(B, 128)
        a_pkc, a_pgc = rnd(B, 512), rnd(B, 512)
        if ratio == 1:
            a_gc = a_pkc = a_pgc = None
        a_pos = torch.tensor([dwl.q_pos0 - (b & 1) for b in range(B)], dtype=torch.int32,
                             device="cuda")
        a_gamma = torch.ones(512, dtype=torch.float32, device="cuda")
        append = lambda: csa2.csa2_append(a_pos, a_kc, a_gc, a_wn, a_pkc, a_pgc, a_gamma, None,
                                          None, a_ki, drun.rope_cos, drun.rope_sin, drun.z_codes,
                                          drun.z_scales, drun.ki_codes, drun.ki_scales,
                                          drun.w_codes, drun.w_scale, ratio=ratio,
                                          z_format=z_format)
        for _ in range(max(args.warmup, 3)):
            append()
        ams = time_events(append, max(args.steps, 20), stream)
        log(f"{key} append: {ams * 1e3:.2f} us per call (B={B})")
        result[key]["append"] = {
            "workload": f"csa2_append B={B}: one token per request at position 131071 or "
                        "131070 " + ("(half close a pair)" if ratio == 2 else "(each writes its "
                                     "entry)") + ", given index keys",
            "us_per_call": ams * 1e3,
            "bytes_per_call": B * (3 * 1024 + 2 * 1024 + 256 + 516 + 340 / 2) if ratio == 2 else
                              B * (2 * 1024 + 256 + 516 + 340),
            "bound": "launch latency (one block of two waves per request)"}
        del drun
        torch.cuda.empty_cache()



def run_pool(args, result, stream, ratio=2):
    """Hierarchical pool and Reindex at the verify-decode shape (B=16 x 6 queries
    at 1,048,570..): the Full layer's scan with and without the pool, and a
    Reindex layer's selection over the pool only.  ratio 2: 524,288 pooled
    entries; ratio 1 (the decoder layers that use the pool): 1,048,576."""
    import dataclasses
    import torch
    import csa2_harness
    import csa2_synth as synth
    import compressed_sparse_attention_csa2_amd as csa2
    wl = synth.workload(4)
    if ratio == 1:
        wl = dataclasses.replace(wl, n_entries=wl.q_pos0 + wl.Tq, ratio=1,
                                 name=wl.name + " ratio 1")
    key = "hierarchical" if ratio == 2 else "hierarchical_ratio1"
    B, Tq, N = wl.B, wl.Tq, wl.n_entries
    log(f"generating index keys: {wl.name}")
    t0 = time.time()
    u8 = torch.uint8
    kc = torch.zeros(B, N, 64, dtype=u8, device="cuda")
    ks = torch.zeros(B, N, 4, dtype=u8, device="cuda")
    for b in range(B):
        for j0 in range(0, N, 1 << 16):
            n = min(1 << 16, N - j0)
            k = csa2_harness.up(wl.ki_rows(b, j0, n))
            csa2.csa2_encode_fp4_rows(k, kc[b, j0:j0 + n].view(n, 64), ks[b, j0:j0 + n].view(n, 4))
            del k
    qI, wI = csa2_harness.up(wl.qI()), csa2_harness.up(wl.wI())
    qI2 = csa2_harness.up(synth.normal(wl.seed, 901, (B, Tq, 32, 128)))     # a Reindex layer's query
    wI2 = csa2_harness.up(synth.normal(wl.seed, 902, (B, Tq, 32), mul=1.0 / 64.0, dtype="f32"))
    q0 = torch.full((B,), wl.q_pos0, dtype=torch.int32, device="cuda")
    ne = torch.full((B,), N, dtype=torch.int32, device="cuda")
    i32 = torch.int32
    idx = torch.empty(B, Tq, 512, dtype=i32, device="cuda")
    cnt = torch.empty(B, Tq, dtype=i32, device="cuda")
    pool = torch.empty(B, Tq, csa2.POOL_BLOCKS, dtype=i32, device="cuda")
    pcnt = torch.empty(B, Tq, dtype=i32, device="cuda")
    idx2, cnt2 = torch.empty_like(idx), torch.empty_like(cnt)
    ws_t = csa2.workspace(csa2.OP_INDEX_TOPK, B, Tq, 64, N)
    ws_p = csa2.workspace(csa2.OP_INDEX_POOL, B, Tq, 64, N)
    ws_r = csa2.workspace(csa2.OP_REINDEX, B, Tq, 64, N)
    torch.cuda.synchronize()
    log(f"index keys resident ({time.time() - t0:.1f} s)")
    full = lambda: csa2.csa2_index_topk(q0, ne, qI, wI, kc, ks, idx, cnt, ws_t, ratio=ratio)
    fpool = lambda: csa2.csa2_index_pool(q0, ne, qI, wI, kc, ks, idx, cnt, pool, pcnt, ws_p,
                                         ratio=ratio)
    reidx = lambda: csa2.csa2_reindex_topk(q0, ne, qI2, wI2, kc, ks, pool, pcnt, idx2, cnt2, ws_r,
                                           ratio=ratio)
    for f in (full, fpool, reidx):
        f()
    torch.cuda.synchronize()
    t_full = time_events(full, args.steps, stream)
    t_pool = time_events(fpool, args.steps, stream)
    t_re = time_events(reidx, args.steps, stream)
    rows = B * Tq
    cand = float(pcnt.sum().item()) * 8
    log(f"{key}: full select {t_full:.4f} ms, with pool {t_pool:.4f} ms, reindex {t_re:.4f} ms")
    gather = cand * 68.0                   # the pool's index keys, gathered per query row
    result[key] = {
        "workload": f"verify-decode shape: B={B} x {Tq} queries at {wl.q_pos0}.., {N} entries "
                    f"at compression ratio {ratio} (lognormal keys, 1% exact duplicates); Full "
                    "layer with the pool, then a Reindex layer's own query over the pool",
        "full_select_ms": t_full, "full_select_with_pool_ms": t_pool, "reindex_select_ms": t_re,
        "candidates_per_row": {"full": N, "reindex": cand / rows},
        "reindex_roofline": {"bound": "hbm", "bytes_per_launch": gather,
                             "achieved": gather / (t_re * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                             "unit": "GB/s", "frac": gather / (t_re * 1e-3) / PEAK_HBM},
    }
    del kc, ks, ws_t, ws_p, ws_r
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
