"""GPU vs oracle parity for favor_attention, through the C ABI.

Bar: per-(b, h) relative Frobenius error <= 1e-4 for float32 inputs and
<= 2e-2 for bf16 inputs.  Small and ragged shapes are compared on every
element; the full-size long-sequence workloads on sampled rows that the
oracle computes one by one."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O
from tests.gpu_util import TOL, from_device, problem, slice_rel_err

pytestmark = pytest.mark.gpu


def _paths(B, H, L, d, m, dtype, kind, causal):
    paths = ["generic"]
    if F.favor_attention_resolve_path(B, H, L, d, m, dtype, kind, causal) == "mfma":
        paths.append("mfma")
    return paths


def _run(dev, kind, causal, path):
    out = F.favor_attention(*dev, kind=kind, causal=causal, path=path)
    torch.cuda.synchronize()
    return from_device(out)


SMALL = [
    # B, H, L, d, m, dtype
    (1, 1, 1, 16, 64, "f32"),
    (1, 2, 7, 16, 16, "f32"),
    (2, 1, 33, 64, 64, "f32"),
    (1, 1, 100, 64, 40, "f32"),
    (1, 1, 1, 64, 256, "bf16"),
    (2, 2, 31, 64, 64, "bf16"),
    (1, 3, 257, 64, 256, "bf16"),
    (1, 1, 1000, 64, 128, "bf16"),
    (2, 1, 130, 16, 64, "bf16"),
    # MFMA with Omega rows not a multiple of 128 (6 and 5 waves per key block)
    (1, 2, 200, 64, 96, "bf16"),
    (1, 1, 150, 64, 160, "bf16"),
    # the fewest Omega rows on MFMA (one wave per block)
    (2, 1, 70, 64, 32, "bf16"),
    # bidirectional MFMA readout summing 4 key-split partials (4 tiles of
    # 128 keys, the last ragged); 1 x 3 x 257 sums 3, 1 x 2 x 200 (m = 96)
    # sums 2, and 1 x 1 x 1000 goes through the split-sum kernel
    (1, 2, 500, 64, 256, "bf16"),
    # m = 512: the bidirectional MFMA readout in two feature passes (the
    # causal and float32 cases run on the generic kernels)
    (1, 2, 300, 64, 512, "bf16"),
]


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[f"{s[0]}x{s[1]}x{s[2]}_d{s[3]}_m{s[4]}_{s[5]}" for s in SMALL])
def test_small_full(shape, kind, causal):
    B, H, L, d, m, dtype = shape
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=L)
    ref = O.favor_attention(q, k, v, W, kind, causal)
    for path in _paths(B, H, L, d, m, dtype, kind, causal):
        got = _run(dev, kind, causal, path)
        ok = np.isfinite(ref).all(axis=-1)
        if kind == "relu":
            # rows with phi(q).phi(K) == 0 are 0/0 on both sides
            assert np.array_equal(ok, np.isfinite(got).all(axis=-1)), path
            got, ref_ = got * ok[..., None], np.where(ok[..., None], ref, 0.0)
        else:
            assert ok.all()
            ref_ = ref
        err = slice_rel_err(np.nan_to_num(got), ref_)
        print(f"[{path}] {shape} {kind} causal={causal} rel={err:.3e}", flush=True)
        assert err <= TOL[dtype], (path, err)


def test_config1_fp32():
    w = I.WORKLOADS["c1"]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal)
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        err = slice_rel_err(_run(dev, w.kind, w.causal, path), ref)
        print(f"[{path}] c1 rel={err:.3e}", flush=True)
        assert err <= 1e-4


@pytest.mark.parametrize("name", ["c2_trig", "c2_relu"])
def test_config2_full(name):
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal, workers=O.default_workers())
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        err = slice_rel_err(_run(dev, w.kind, w.causal, path), ref)
        print(f"[{path}] {name} rel={err:.3e}", flush=True)
        assert err <= 2e-2


@pytest.mark.parametrize("name", ["c3_causal", "head", "c4_bidir", "c4_causal", "pos_bidir", "pos_causal"])
def test_full_size_sampled_rows(name):
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype, norm_shells=w.norm_shells)
    rows = I.sample_rows(w.L, 256, seed=0)
    ref = O.favor_rows(q, k, v, W, w.kind, w.causal, rows)
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        got = _run(dev, w.kind, w.causal, path)[..., rows, :]
        err = slice_rel_err(got, ref)
        print(f"[{path}] {name} sampled rel={err:.3e}", flush=True)
        assert err <= 2e-2


@pytest.mark.parametrize("kind", ["trig", "positive"])
@pytest.mark.parametrize("BH", [(1, 4), (4, 8)], ids=["B1H4", "B4H8"])
def test_m512_long_sampled_rows(BH, kind):
    # the top of the pages' feature grid at a long sequence: L4096, m = 512,
    # bidirectional (MFMA readout in two feature passes).  B1 H4 runs
    # 4-wave readout blocks, B4 H8 the 8-wave ones.
    (B, H), L, d, m = BH, 4096, 64, 512
    assert F.favor_attention_resolve_path(B, H, L, d, m, "bf16", kind, False) == "mfma"
    dev, (q, k, v), W = problem(B, H, L, d, m, "bf16", seed=512)
    rows = I.sample_rows(L, 256, seed=0)
    ref = O.favor_rows(q, k, v, W, kind, False, rows)
    for path in _paths(B, H, L, d, m, "bf16", kind, False):
        got = _run(dev, kind, False, path)[..., rows, :]
        err = slice_rel_err(got, ref)
        print(f"[{path}] m512 {kind} sampled rel={err:.3e}", flush=True)
        assert err <= 2e-2


def test_causal_matches_masked_form_c3_rows():
    # config 3 is also checked against the explicitly masked quadratic form
    w = I.WORKLOADS["c3_causal"]
    dev, (q, k, v), W = problem(1, 2, w.L, w.d, w.m, w.dtype)
    rows = np.array([0, 1, 2, 3, 511, 512, 1023, 2047, 4094, 4095])
    ref = O.favor_quadratic_rows(q, k, v, W, "trig", True, rows)
    for path in _paths(1, 2, w.L, w.d, w.m, w.dtype, "trig", True):
        got = _run(dev, "trig", True, path)[..., rows, :]
        assert slice_rel_err(got, ref) <= 2e-2


@pytest.mark.parametrize("causal", [False, True])
def test_deterministic(causal):
    dev, _, _ = problem(2, 4, 2048, 64, 256, "bf16", seed=11)
    for path in _paths(2, 4, 2048, 64, 256, "bf16", "trig", causal):
        a = F.favor_attention(*dev, kind="trig", causal=causal, path=path)
        b = F.favor_attention(*dev, kind="trig", causal=causal, path=path)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), path


def test_workspace_contents_ignored():
    dev, (q, k, v), W = problem(1, 2, 300, 64, 256, "bf16", seed=3)
    ref = O.favor_attention(q, k, v, W, "trig", True)
    for path in _paths(1, 2, 300, 64, 256, "bf16", "trig", True):
        need = F.favor_attention_workspace_bytes(1, 2, 300, 64, 256, "bf16", "trig", True, path)
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage
        out = F.favor_attention(*dev, kind="trig", causal=True, path=path, workspace=ws)
        torch.cuda.synchronize()
        assert slice_rel_err(from_device(out), ref) <= 2e-2


def test_nonfinite_input_propagates():
    dev, _, _ = problem(1, 1, 64, 64, 256, "bf16", seed=4)
    q, k, v, w = dev
    v = v.clone()
    v[0, 0, 5, 3] = float("nan")
    for path in _paths(1, 1, 64, 64, 256, "bf16", "trig", False):
        out = F.favor_attention(q, k, v, w, kind="trig", path=path)
        torch.cuda.synchronize()
        assert torch.isnan(out[0, 0, :, 3]).all()


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
@pytest.mark.parametrize("which", ["k", "v"])
def test_causal_nonfinite_last_token_stays_local(which, kind):
    # The causal output of token i depends on tokens j <= i only.  A NaN in
    # the last token's key or value reaches that token's output.  The
    # float32 path keeps every earlier output bit for bit; the MFMA path
    # multiplies a chunk's value rows by masked scores, so the NaN may also
    # reach the earlier tokens of its own 32-token chunk (NaN * 0), but no
    # token of an earlier chunk.  L = 70 ends in a ragged chunk [64, 96).
    B, H, L, d, m = 1, 2, 70, 64, 256
    chunk0 = (L - 1) // 32 * 32
    dev, _, _ = problem(B, H, L, d, m, "bf16", seed=L)
    q, k, v, w = dev
    bad = {"k": k, "v": v}[which].clone()
    bad[:, :, L - 1, 5] = float("nan")
    args = (bad, v) if which == "k" else (k, bad)
    for path in _paths(B, H, L, d, m, "bf16", kind, True):
        clean = F.favor_attention(q, k, v, w, kind=kind, causal=True, path=path)
        out = F.favor_attention(q, *args, w, kind=kind, causal=True, path=path)
        torch.cuda.synchronize()
        keep = L - 1 if path == "generic" else chunk0
        fin = torch.isfinite(clean.float()).all(dim=-1)[:, :, :keep]   # ReLU may have 0/0 rows
        assert torch.equal(out[:, :, :keep][fin].view(torch.int16), clean[:, :, :keep][fin].view(torch.int16)), path
        if not (kind == "relu" and which == "k"):
            # (the device's ReLU features are max(P, 0) with IEEE maxNum: a
            # NaN projection gives the feature 0, so a NaN key drops out)
            assert torch.isnan(out[:, :, L - 1]).any(), path


def test_profile_reports_kernels():
    dev, _, _ = problem(1, 2, 512, 64, 256, "bf16")
    for path in _paths(1, 2, 512, 64, 256, "bf16", "trig", False):
        phases = F.favor_profile_attention(*dev, kind="trig", path=path, iters=3)
        assert phases and all(ms > 0 for _, ms in phases)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["trig", "relu"])
def test_profile_output_matches_call(kind, causal):
    # favor_profile_attention repeats kernels back-to-back; its output must
    # still be the call's result (no phase may be repeated on its own output)
    dev, _, _ = problem(1, 2, 300, 64, 256, "bf16", seed=9)
    for path in _paths(1, 2, 300, 64, 256, "bf16", kind, causal):
        ref = F.favor_attention(*dev, kind=kind, causal=causal, path=path)
        out = torch.empty_like(ref)
        F.favor_profile_attention(*dev, kind=kind, causal=causal, path=path, iters=4, out=out)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), out.view(torch.int16)), path
