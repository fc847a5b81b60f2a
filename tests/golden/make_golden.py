"""Writes tests/golden/*.json from the oracle alone (no GPU code is imported).

The pages print no worked numerical example for the KDN layer, so the only
stored values here are oracle outputs on the seeded small workloads; they pin
the oracle against later edits of itself (the closed forms and special cases
in test_oracle_pins.py pin it against the mathematics).

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from kdn_inputs import config_inputs  # noqa: E402


def sample(cfg_index, variant, path, T=None):
    over = {} if T is None else {"T": T}
    inp = config_inputs(cfg_index, variant=variant, **over)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant)
    B, H, Tn, dv = out["o"].shape
    rng = np.random.default_rng(0)
    idx = [(int(b), int(h), int(t), int(j)) for b, h, t, j in zip(
        rng.integers(0, B, 64), rng.integers(0, H, 64), rng.integers(0, Tn, 64),
        rng.integers(0, dv, 64))]
    rec = {
        "what": "oracle outputs on the seeded workload; regression pin of the oracle",
        "workload": {"config_index": cfg_index, "variant": variant, "T": Tn},
        "o_samples": [[*i, float(out["o"][i])] for i in idx],
        "S_T_row0": out["S_T"][0, 0, 0].tolist(),
        "lambda_T": np.ravel(out["lambda_T"]).tolist(),
    }
    with open(path, "w") as f:
        json.dump(rec, f)


if __name__ == "__main__":
    sample(0, "isotropic", os.path.join(HERE, "oracle_iso_f32_B1_H2_T256_d32.json"))
    sample(1, "diagonal", os.path.join(HERE, "oracle_diag_f32_B2_H4_T256_d64.json"), T=256)
