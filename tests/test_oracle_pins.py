"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle_pins as P
from synth.workloads import FITCHECK


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _local_cases():
    with open(os.path.join(P.GOLDEN, "kvbridge_local_evidence.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _local_cases(), ids=lambda c: c["name"])
def test_kvbridge_local_evidence_geometry(case):
    """The KVBridge README's three synthetic geometries: every true layer recovered, holdout
    R^2 above 0.99999 and within a factor 3 of the printed 1 - R^2."""
    cfg = FITCHECK.replace(cid=100 + case["L_src"], L_src=case["L_src"], L_tgt=case["L_tgt"],
                           H=case["H"], d=case["d"], T=case["T"])
    fit, pr, r2 = P.run_fitcheck(cfg)
    assert np.array_equal(fit["layer_sel"], pr["draws"]["true_sel"])
    assert r2.min() > 0.99999
    printed = 1.0 - case["holdout_r2"]
    ours = 1.0 - r2.mean()
    assert printed / 3 < ours < printed * 3, (ours, printed)
