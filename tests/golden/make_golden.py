"""Write tests/golden/oracle_workload0.json: digests of the oracle's outputs on the
T=256, H=16 prefill workload (derived index keys).  Calls only oracle/ and the
seeded input generator; run it after a deliberate, justified oracle change."""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import csa2_synth  # noqa: E402
from oracle.reference import PrefillReference  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    wl = csa2_synth.workload(0)
    ref = PrefillReference(wl)
    w_codes, w_scale = ref.window_full()
    rows = np.arange(wl.Tq)
    r = ref.rows(rows)
    return {
        "workload": wl.name,
        "z_codes": digest(ref.z_codes), "z_scales": digest(ref.z_scales),
        "ki_codes": digest(ref.ki_codes), "ki_scales": digest(ref.ki_scales),
        "w_codes": digest(w_codes), "w_scale": digest(w_scale),
        "idx": digest(r["idx"]), "cnt": digest(r["cnt"]),
        "O_bf16": digest(r["O_bf16"]),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_workload0.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
