"""Golden fixtures: the numbers the pages print, and digests that freeze the oracle's
output on the T=256 prefill workload (regenerated only by tests/golden/make_golden.py)."""
import json
import math
import os

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_page_constants_agree_with_the_oracle(orc):
    c = load("page_constants.json")
    v = {k: e["value"] for k, e in c.items() if not k.startswith("_")}
    assert v["window"] + v["topk"] == v["attended_rows"]
    assert v["heads"] * v["latent_dim"] == 32768
    assert v["indexer_heads"] * v["indexer_dim"] == v["indexer_weight_scale_sq"]
    # an index key encoded by the oracle occupies the printed 68 bytes
    codes, scales = orc.fp4_encode(np.random.default_rng(0).standard_normal((1, 128)))
    assert codes.nbytes + scales.nbytes == v["index_key_bytes"]
    assert v["latent_dim"] * 4 // 8 + v["latent_dim"] // 16 == v["main_entry_bytes_pages_format"]
    assert v["main_entry_bytes_pages_format"] + v["index_key_bytes"] == v["pair_bytes"]
    assert (3 / 2 + 1) * v["pair_bytes"] == v["bytes_per_token"]
    assert abs(math.sqrt(v["latent_dim"]) - v["value_bound"]) < 0.05
    assert v["latent_dim"] - v["rope_lo"] == 64 and v["indexer_dim"] - v["index_rope_lo"] == 64


def test_oracle_digests_on_the_small_prefill():
    from tests.golden.make_golden import compute
    assert compute() == load("oracle_workload0.json")
