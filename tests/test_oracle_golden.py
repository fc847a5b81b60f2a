"""Regression pin: the oracle reproduces the values tests/golden/make_golden.py
stored from it (the pages print no worked example of their own)."""
import json
import os

import numpy as np
import pytest

import oracle
from kdn_inputs import config_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("fname", ["oracle_iso_f32_B1_H2_T256_d32.json",
                                   "oracle_diag_f32_B2_H4_T256_d64.json"])
def test_oracle_matches_stored_values(fname):
    with open(os.path.join(GOLDEN, fname)) as f:
        rec = json.load(f)
    wl = rec["workload"]
    inp = config_inputs(wl["config_index"], variant=wl["variant"], T=wl["T"])
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], wl["variant"])
    for b, h, t, j, val in rec["o_samples"]:
        assert out["o"][b, h, t, j] == pytest.approx(val, rel=1e-12, abs=1e-14)
    np.testing.assert_allclose(out["S_T"][0, 0, 0], rec["S_T_row0"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.ravel(out["lambda_T"]), rec["lambda_T"], rtol=1e-12)
