"""GPU checks of the saved-forward pair: favor_attention_train's row
normaliser D_ii = phi(q_i) . sum_j phi(k_j) (j <= i when causal) against
the oracle's feature maps, its output against favor_attention's, and
favor_attention_backward_saved's gradients against the oracle.

Bar: as the other parity tests -- per-(b, h) relative Frobenius error
<= 1e-4 for float32 inputs and <= 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O
from tests.gpu_util import TOL, from_device, problem, to_device

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, L, d, m, dtype
    (1, 2, 33, 16, 64, "f32"),
    (2, 1, 100, 64, 40, "f32"),
    (2, 2, 31, 64, 64, "bf16"),
    (1, 3, 257, 64, 256, "bf16"),
    (2, 1, 70, 64, 32, "bf16"),
]
IDS = [f"{s[0]}x{s[1]}x{s[2]}_d{s[3]}_m{s[4]}_{s[5]}" for s in SHAPES]


def _paths(shape, kind, causal):
    B, H, L, d, m, dtype = shape
    paths = ["generic"]
    if F.favor_attention_resolve_path(B, H, L, d, m, dtype, kind, causal) == "mfma":
        paths.append("mfma")
    return paths


def _fwd_paths(shape, kind, causal):
    # the forward families, the small two-launch path included
    B, H, L, d, m, dtype = shape
    paths = _paths(shape, kind, causal)
    try:
        F.favor_attention_resolve_path(B, H, L, d, m, dtype, kind, causal, "small")
        paths.append("small")
    except F.FavorError:
        pass
    return paths


def _oracle_den(q, k, W, kind, causal):
    """sum_j phi(q_i) . phi(k_j) over j (j <= i when causal), per (b, h)."""
    pq, pk = O.feature_map(q, W, kind), O.feature_map(k, W, kind)
    if causal:
        return np.einsum("...lf,...lf->...l", pq, np.cumsum(pk, axis=-2))
    return np.einsum("...lf,...f->...l", pq, pk.sum(axis=-2))


def _rel(got, ref):
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    return max(np.linalg.norm(g[i] - r[i]) / np.linalg.norm(r[i]) for i in range(g.shape[0]))


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_forward_den(shape, kind, causal):
    B, H, L, d, m, dtype = shape
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=3)
    ref = _oracle_den(q, k, W, kind, causal)
    with np.errstate(invalid="ignore", divide="ignore"):
        out_ref = O.favor_attention(q, k, v, W, kind, causal)
    if not np.isfinite(out_ref).all():
        pytest.skip("0/0 row in the forward (ReLU)")
    for path in _fwd_paths(shape, kind, causal):
        out, den = F.favor_attention(*dev, kind=kind, causal=causal, path=path, den=True)
        plain = F.favor_attention(*dev, kind=kind, causal=causal, path=path)
        torch.cuda.synchronize()
        err = _rel(den.cpu().numpy().astype(np.float64), ref)
        print(f"[{path}] {shape} {kind} causal={causal} den rel = {err:.2e}", flush=True)
        assert err <= TOL[dtype], (path, err)
        # requesting den leaves the output unchanged
        assert torch.equal(out.view(torch.int16) if dtype == "bf16" else out,
                           plain.view(torch.int16) if dtype == "bf16" else plain)


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
def test_forward_den_m512(kind):
    # m = 512: the bidirectional MFMA readout takes its features in two
    # passes; its row normalisers against the oracle's feature maps
    B, H, L, d, m, dtype = 1, 2, 300, 64, 512, "bf16"
    assert F.favor_attention_resolve_path(B, H, L, d, m, dtype, kind, False) == "mfma"
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=7)
    with np.errstate(invalid="ignore", divide="ignore"):
        if not np.isfinite(O.favor_attention(q, k, v, W, kind, False)).all():
            pytest.skip("0/0 row in the forward (ReLU)")
    ref = _oracle_den(q, k, W, kind, False)
    for path in ("generic", "mfma"):
        out, den = F.favor_attention(*dev, kind=kind, causal=False, path=path, den=True)
        torch.cuda.synchronize()
        err = _rel(den.cpu().numpy().astype(np.float64), ref)
        print(f"[{path}] m512 {kind} den rel = {err:.2e}", flush=True)
        assert err <= TOL[dtype], (path, err)


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES[2:] + [(4, 8, 1024, 64, 256, "bf16")],
                         ids=IDS[2:] + ["4x8x1024_d64_m256_bf16"])
def test_backward_saved(shape, kind, causal):
    B, H, L, d, m, dtype = shape
    for s in range(3, 23):
        dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=s)
        with np.errstate(invalid="ignore", divide="ignore"):
            if np.isfinite(O.favor_attention(q, k, v, W, kind, causal)).all():
                break
    else:
        pytest.skip("no draw without 0/0 rows")
    gs, g64 = I.output_grads(B, H, L, d, dtype, seed=s)
    g_dev = to_device(gs, dtype)
    ref = O.favor_attention_grad(q, k, v, W, g64, kind, causal, workers=O.default_workers())
    for path in _paths(shape, kind, causal):
        out, den = F.favor_attention(*dev, kind=kind, causal=causal, path=path, den=True)
        got = F.favor_attention_backward(*dev, g_dev, kind=kind, causal=causal, path=path,
                                         saved=(out, den))
        torch.cuda.synchronize()
        errs = []
        for x, r in zip(got, ref):
            x = from_device(x).reshape(-1, L, d)
            rr = r.reshape(-1, L, d)
            sc = ref[2].reshape(-1, L, d)
            e = 0.0
            for i in range(x.shape[0]):
                nr = np.linalg.norm(rr[i])
                e = max(e, np.linalg.norm(x[i] - rr[i]) / (nr if nr > 1e-6 * np.linalg.norm(sc[i]) else np.linalg.norm(sc[i])))
            errs.append(e)
        print(f"[{path}] {shape} {kind} causal={causal} saved dq/dk/dv rel = "
              + " ".join(f"{e:.2e}" for e in errs), flush=True)
        for name, e in zip(("dq", "dk", "dv"), errs):
            assert e <= TOL[dtype], (path, name, e)


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_function(dtype, causal, kind):
    # loss.backward() through the autograd wrapper gives the gradients of the
    # direct backward call (within the bar), the forward gives
    # favor_attention's output bit for bit, and the gradients stay within
    # the bar of the oracle's
    B, H, L, d, m = 2, 2, 200, 64, 64
    for s in range(5, 25):
        dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=s)
        with np.errstate(invalid="ignore", divide="ignore"):
            if np.isfinite(O.favor_attention(q, k, v, W, kind, causal)).all():
                break
    else:
        pytest.skip("no draw without 0/0 rows")
    gs, g64 = I.output_grads(B, H, L, d, dtype, seed=s)
    g_dev = to_device(gs, dtype)
    leaves = [x.clone().requires_grad_(True) for x in dev[:3]]
    out = F.favor_attention_fn(*leaves, dev[3], kind=kind, causal=causal)
    out.backward(g_dev)
    want_out = F.favor_attention(*dev, kind=kind, causal=causal)
    want = F.favor_attention_backward(*dev, g_dev, kind=kind, causal=causal)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t)
    assert torch.equal(bits(out.detach()), bits(want_out))
    ref = O.favor_attention_grad(q, k, v, W, g64, kind, causal, workers=O.default_workers())
    for name, leaf, w, r in zip(("dq", "dk", "dv"), leaves, want, ref):
        a = leaf.grad.float()
        b = w.float()
        assert torch.linalg.norm(a - b) <= TOL[dtype] * torch.linalg.norm(b), name
        got = from_device(leaf.grad).reshape(-1, L, d)
        rr = r.reshape(-1, L, d)
        sc = ref[2].reshape(-1, L, d)   # dV's scale where a slice is ~0
        e = 0.0
        for i in range(got.shape[0]):
            nr = np.linalg.norm(rr[i])
            den = nr if nr > 1e-6 * np.linalg.norm(sc[i]) else np.linalg.norm(sc[i])
            e = max(e, np.linalg.norm(got[i] - rr[i]) / den)
        assert e <= TOL[dtype], (name, e)


def test_forward_den_full_grid_trig():
    # the headline shape, where the trig readout runs 16 waves of 32 queries
    # per block: its row normalisers (the query rows reloaded in the
    # epilogue) against the oracle's feature maps, and the output unchanged
    # by asking for them
    B, H, L, d, m, dtype = 4, 8, 4096, 64, 256, "bf16"
    assert F.favor_attention_resolve_path(B, H, L, d, m, dtype, "trig", False) == "mfma"
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=8)
    ref = _oracle_den(q, k, W, "trig", False)
    out, den = F.favor_attention(*dev, kind="trig", causal=False, path="mfma", den=True)
    plain = F.favor_attention(*dev, kind="trig", causal=False, path="mfma")
    torch.cuda.synchronize()
    err = _rel(den.cpu().numpy().astype(np.float64), ref)
    print(f"[mfma] B4 H8 L4096 trig den rel = {err:.2e}", flush=True)
    assert err <= TOL[dtype], err
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
