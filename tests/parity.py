"""Comparison rules between the HIP path and the oracle.

* Storage codes and scales: bit-exact.
* Selections: counts exact; index sets equal, except boundary swaps -- an
  entry chosen by one side but not the other is allowed only when every such
  entry's oracle fp32 score is within 1e-5 (relative) of the others involved
  (the two sides rank in fp32 with different accumulation orders).  Order is
  ascending, padding -1.
* Attention output (bf16): max |dO| <= 2e-2 and ||dO|| / ||O|| <= 1e-2 against
  the oracle's double result, on the same selected rows.
"""
import numpy as np

MAX_ABS = 2e-2
REL_RMS = 1e-2
SWAP_REL = 1e-5


def bf16_to_f64(x):
    return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_selection(g_idx, g_cnt, o_idx, o_cnt, o_scores=None):
    """one query row; returns number of boundary swaps; raises AssertionError on violation"""
    assert int(g_cnt) == int(o_cnt), f"count {g_cnt} != oracle {o_cnt}"
    c = int(o_cnt)
    g = np.asarray(g_idx)
    assert np.all(g[c:] == -1), "padding must be -1"
    sel = g[:c]
    assert np.all(np.diff(sel) > 0), "selection must be strictly ascending"
    a = set(sel.tolist())
    b = set(np.asarray(o_idx)[:c].tolist())
    if a == b:
        return 0
    only_g, only_o = sorted(a - b), sorted(b - a)
    assert len(only_g) == len(only_o)
    assert o_scores is not None, "selections differ and no oracle scores to judge the swap"
    vals = np.array([o_scores[j] for j in only_g + only_o], np.float64)
    spread = vals.max() - vals.min()
    scale = np.abs(vals).max()
    assert spread <= SWAP_REL * scale, (
        f"non-boundary swap: gpu-only {only_g[:4]} oracle-only {only_o[:4]} "
        f"scores {vals[:8]} spread {spread:.3e}")
    return len(only_g)


def attention_error(gpu_bf16, oracle_f64):
    g = bf16_to_f64(gpu_bf16)
    d = g - oracle_f64
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(oracle_f64), 1e-30))


def check_attention(gpu_bf16, oracle_f64, what=""):
    mx, rel = attention_error(gpu_bf16, oracle_f64)
    assert mx <= MAX_ABS and rel <= REL_RMS, f"{what}: max|dO|={mx:.3e} rel_rms={rel:.3e}"
    return mx, rel


def oracle_threads() -> int:
    """worker threads for oracle evaluations: the C oracle releases the GIL inside
    each call and keeps no shared state, so disjoint rows run in parallel"""
    import os
    return max(1, min(16, os.cpu_count() or 1))


def parallel_map(fn, items, threads=None):
    """[fn(x) for x in items], evaluated on a thread pool (order kept)"""
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    with ThreadPoolExecutor(max_workers=threads or oracle_threads()) as ex:
        return list(ex.map(fn, items))


def prefill_rows_parallel(ref, rows, chunk=8, **kw):
    """PrefillReference.rows over many rows in parallel chunks; the window must
    already be encoded (ref.window_full()), so no call mutates the reference"""
    import numpy as np
    rows = np.asarray(rows, np.int64)
    parts = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    res = parallel_map(lambda r: ref.rows(r, **kw), parts)
    out = {}
    for k in res[0]:
        vals = [r[k] for r in res]
        out[k] = None if vals[0] is None else np.concatenate(vals)
    return out
