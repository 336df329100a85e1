"""Hand-derived worked examples (tests/golden/*.json) against the fp64 oracle.

Each fixture states its derivation from the equations of
"解析 FlashAttention（3）：FlashAttention-v1 反向传播" in its own text.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden(path):
    g = json.load(open(path))
    arr = lambda n: np.array(g[n], dtype=np.float64)[None, None]
    r = oracle.reference(arr("Q"), arr("K"), arr("V"), arr("dO"), g["tau"], g["causal"], g["softcap"])
    for name in ("O", "LSE", "D", "dQ", "dK", "dV"):
        np.testing.assert_allclose(r[name][0, 0], np.array(g[name], dtype=np.float64), rtol=0, atol=1e-15,
                                   err_msg=name)


def test_fixtures_present():
    assert len(GOLDEN) >= 2
