"""The oracle against hand-derived d = 1 examples (tests/golden/handworked.json)."""
import json
import os

import numpy as np
import pytest

from oracle import favor_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "handworked.json")))["cases"]


@pytest.mark.filterwarnings("ignore:invalid value")
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_handworked(case):
    W = np.array(case["omega"])
    q, k, v = (np.array(case[n]) for n in ("q", "k", "v"))
    for mode in ("bidirectional", "causal"):
        if mode not in case:
            continue
        want = np.array([[np.nan if x is None else x for x in row] for row in case[mode]])
        got = O.favor_attention(q, k, v, W, case["kind"], causal=(mode == "causal"))
        assert np.array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        assert np.allclose(got[ok], want[ok], rtol=0, atol=case["atol"]), (got, want)
