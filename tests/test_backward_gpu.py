"""GPU vs oracle parity for favor_attention_backward, through the C ABI.

Bar: per-(b, h) relative Frobenius error of each of dQ, dK, dV <= 1e-4
for float32 inputs and <= 2e-2 for bf16 inputs, against the float64
oracle gradients on the same stored inputs.  Problems whose forward has a
0/0 row (possible for the ReLU map) are redrawn: such a row makes every
key gradient of its head NaN on both sides."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O
from tests.gpu_util import TOL, from_device, problem, slice_rel_err, to_device

pytestmark = pytest.mark.gpu

SMALL = [
    # B, H, L, d, m, dtype
    (1, 1, 1, 16, 64, "f32"),
    (1, 2, 7, 16, 16, "f32"),
    (2, 1, 33, 64, 64, "f32"),
    (1, 1, 100, 64, 40, "f32"),
    (2, 2, 31, 64, 64, "bf16"),
    (1, 3, 257, 64, 256, "bf16"),
    (2, 1, 130, 16, 64, "bf16"),
    # MFMA with Omega rows not a multiple of 128 (6 and 5 waves per key block)
    (1, 2, 200, 64, 96, "bf16"),
    (1, 1, 150, 64, 160, "bf16"),
    # MFMA edge cases: one token; the fewest Omega rows (one wave per block); m = 128
    (1, 2, 1, 64, 64, "bf16"),
    (2, 1, 70, 64, 32, "bf16"),
    (1, 1, 300, 64, 128, "bf16"),
]


def _grad_problem(shape, kind, causal, seed):
    B, H, L, d, m, dtype = shape
    for s in range(seed, seed + 20):
        dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=s)
        with np.errstate(invalid="ignore", divide="ignore"):
            ok = np.isfinite(O.favor_attention(q, k, v, W, kind, causal)).all()
        if ok:
            gs, g64 = I.output_grads(B, H, L, d, dtype, seed=s)
            return dev, (q, k, v), W, to_device(gs, dtype), g64
    pytest.skip("no draw without 0/0 rows")


def _grad_err(got, ref, scale_ref):
    """max over (b, h) slices of |got - ref|_F / |ref|_F; a slice whose
    reference gradient is zero (one token: dQ = dK = 0) is measured against
    the slice's dV norm instead."""
    g = got.reshape(-1, *got.shape[-2:])
    r = ref.reshape(-1, *ref.shape[-2:])
    sc = scale_ref.reshape(-1, *scale_ref.shape[-2:])
    errs = []
    for i in range(g.shape[0]):
        nr, ns = np.linalg.norm(r[i]), np.linalg.norm(sc[i])
        errs.append(np.linalg.norm(g[i] - r[i]) / (nr if nr > 1e-6 * ns else ns))
    return float(max(errs))


def _paths(shape, kind, causal):
    B, H, L, d, m, dtype = shape
    paths = ["generic"]
    if F.favor_attention_backward_resolve_path(B, H, L, d, m, dtype, kind, causal) == "mfma":
        paths.append("mfma")
    return paths


def _check(shape, kind, causal, seed=0, workers=None, paths=None):
    dtype = shape[-1]
    dev, (q, k, v), W, g_dev, g64 = _grad_problem(shape, kind, causal, seed)
    ref = O.favor_attention_grad(q, k, v, W, g64, kind, causal, workers=workers)
    for path in paths or _paths(shape, kind, causal):
        got = F.favor_attention_backward(*dev, g_dev, kind=kind, causal=causal, path=path)
        torch.cuda.synchronize()
        errs = [_grad_err(from_device(x), r, ref[2]) for x, r in zip(got, ref)]
        print(f"[{path}] {shape} {kind} causal={causal} dq/dk/dv rel = "
              + " ".join(f"{e:.2e}" for e in errs), flush=True)
        for name, e in zip(("dq", "dk", "dv"), errs):
            assert e <= TOL[dtype], (path, name, e)


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[f"{s[0]}x{s[1]}x{s[2]}_d{s[3]}_m{s[4]}_{s[5]}" for s in SMALL])
def test_backward_small(shape, kind, causal):
    _check(shape, kind, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_config2_shape(causal):
    # the B8 H8 L1024 d64 m256 bf16 workload shape
    _check((8, 8, 1024, 64, 256, "bf16"), "trig", causal, workers=O.default_workers())


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
def test_backward_mfma_headline_shape(kind):
    # B4 H8 L4096 d64 m256 bf16 bidirectional (4 token splits per head)
    _check((4, 8, 4096, 64, 256, "bf16"), kind, False, workers=O.default_workers(), paths=["mfma"])


def test_backward_mfma_many_splits():
    # L = 32768 with 8 heads: more splits than the readout sums itself
    _check((1, 8, 32768, 64, 256, "bf16"), "trig", False, workers=O.default_workers(), paths=["mfma"])


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
def test_backward_mfma_causal_headline_shape(kind):
    # B4 H8 L4096 d64 m256 bf16 causal (16 segments of 256 tokens per head)
    _check((4, 8, 4096, 64, 256, "bf16"), kind, True, workers=O.default_workers(), paths=["mfma"])


def test_backward_mfma_causal_many_segments():
    # two heads of 8192 tokens: 64 segments per head, so the prefix and
    # suffix scans run over many segment states
    _check((1, 2, 8192, 64, 256, "bf16"), "trig", True, workers=O.default_workers(), paths=["mfma"])


def test_backward_mfma_causal_segment_scan_remainder():
    # 20 segments per head: the prefix and suffix scans run one batch of 16
    # segments and four one at a time
    _check((1, 2, 2560, 64, 256, "bf16"), "trig", True, workers=O.default_workers(), paths=["mfma"])


def test_backward_config1():
    _check((1, 1, 512, 16, 64, "f32"), "trig", False)


@pytest.mark.parametrize("causal,path", [(True, "generic"), (False, "mfma"), (True, "mfma")])
def test_backward_workspace_contents_ignored(causal, path):
    shape = (1, 2, 300, 64, 256, "bf16")
    dev, (q, k, v), W, g_dev, g64 = _grad_problem(shape, "trig", causal, 3)
    ref = O.favor_attention_grad(q, k, v, W, g64, "trig", causal)
    need = F.favor_attention_backward_workspace_bytes(1, 2, 300, 64, 256, "bf16", "trig", causal, path)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    got = F.favor_attention_backward(*dev, g_dev, kind="trig", causal=causal, workspace=ws,
                                     path=path)
    torch.cuda.synchronize()
    for x, r in zip(got, ref):
        assert slice_rel_err(from_device(x), r) <= 2e-2


@pytest.mark.parametrize("causal", [False, True])
def test_backward_deterministic(causal):
    shape = (2, 2, 600, 64, 128, "bf16")
    dev, _, _, g_dev, _ = _grad_problem(shape, "trig", causal, 4)
    a = F.favor_attention_backward(*dev, g_dev, kind="trig", causal=causal)
    b = F.favor_attention_backward(*dev, g_dev, kind="trig", causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
