"""The estimator-quality sweep on the GPU, at a reduced size: the error
against exact softmax attention falls with m (about 1/sqrt(m): P5), and
orthogonal features are no worse than i.i.d. ones."""
import numpy as np
import pytest

from linear_kernelized_attention_amd import sweep

pytestmark = pytest.mark.gpu


def test_softmax_rows_is_softmax():
    # the comparison target against a direct evaluation on a tiny input
    r = np.random.default_rng(0)
    q, k, v = (r.standard_normal((2, 5, 4)) for _ in range(3))
    rows = np.array([0, 3])
    got = sweep.softmax_rows(q, k, v, rows)
    for h in range(2):
        s = np.exp(q[h] @ k[h].T / 2.0)
        ref = (s / s.sum(1, keepdims=True)) @ v[h]
        np.testing.assert_allclose(got[h], ref[rows], rtol=1e-12)


def test_sweep_trends():
    res = sweep.run(L=1024, H=2, ms=(64, 512), kinds=("positive", "trig"), scales=("x1",),
                    seeds=(0, 1, 2))
    err = {(r["kind"], r["m"], r["features"]): r["rel_err_mean"] for r in res["rows"]}
    for r in res["rows"]:
        print(r, flush=True)
    for kind in ("positive", "trig"):
        for feat in ("orf", "iid"):
            # eight times the features: the error falls by about sqrt(8)
            assert err[(kind, 512, feat)] < err[(kind, 64, feat)] / 1.8
        assert err[(kind, 64, "orf")] <= 1.15 * err[(kind, 64, "iid")]
