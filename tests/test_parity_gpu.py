"""GPU vs oracle parity for favor_attention, through the C ABI.

Bar: per-(b, h) relative Frobenius error and the largest per-row relative
error both <= 1e-4 for float32 inputs and <= 2e-2 for bf16 inputs.  Every
workload is compared on every output row; the two L = 32768 workloads
are also compared on sampled rows that the oracle computes one by one."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O
from tests.gpu_util import TOL, assert_parity, from_device, problem, slice_rel_err, to_device

pytestmark = pytest.mark.gpu


def _paths(B, H, L, d, m, dtype, kind, causal):
    paths = ["generic"]
    for fam in ("mfma", "small"):
        try:
            F.favor_attention_resolve_path(B, H, L, d, m, dtype, kind, causal, fam)
            paths.append(fam)
        except F.FavorError:
            pass
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
    # sums 2, 1 x 1 x 1000 sums 8, and 1 x 1 x 1500 (12 splits) goes
    # through the split-sum kernel
    (1, 2, 500, 64, 256, "bf16"),
    (1, 1, 1500, 64, 256, "bf16"),
    # m = 512: the bidirectional MFMA readout in two feature passes (the
    # causal and float32 cases run on the generic kernels)
    (1, 2, 300, 64, 512, "bf16"),
    # the small path's one-launch kernel at its limits: d = 32 (three value
    # column tiles), m = 128 (16 waves), L = 512 (16 key steps per half);
    # d = 8 (one column tile) with m = 16 (two waves) and a ragged tail;
    # d = 24 with three Omega row tiles
    (1, 1, 512, 32, 128, "f32"),
    (1, 2, 33, 8, 16, "f32"),
    (2, 1, 200, 24, 48, "bf16"),
    # the small path's two launches: past the one-launch kernel's sequence
    # limit, and d and m that are not multiples of 8 and 16
    (1, 1, 700, 16, 64, "f32"),
    (1, 2, 300, 20, 40, "f32"),
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
        assert_parity(np.nan_to_num(got), ref_, TOL[dtype], f"[{path}] {shape} {kind} causal={causal}")


@pytest.mark.parametrize("kind", ["trig", "positive"])
def test_causal_segment_scan_batches(kind):
    # B1 H2 L2560: 20 segments of 128 tokens per head on a grid of a few
    # dozen blocks, so the exclusive segment scan runs one batch of 16
    # segments and then four one at a time
    B, H, L, d, m = 1, 2, 2560, 64, 256
    dev, (q, k, v), W = problem(B, H, L, d, m, "bf16", seed=20)
    ref = O.favor_attention(q, k, v, W, kind, True, workers=O.default_workers())
    got = _run(dev, kind, True, "mfma")
    assert_parity(got, ref, 2e-2, f"[mfma] {kind} causal, 20 segments")


def test_config1_fp32():
    w = I.WORKLOADS["c1"]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal)
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        assert_parity(_run(dev, w.kind, w.causal, path), ref, 1e-4, f"[{path}] c1")


@pytest.mark.parametrize("name", ["c2_trig", "c2_relu"])
def test_config2_full(name):
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal, workers=O.default_workers())
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        assert_parity(_run(dev, w.kind, w.causal, path), ref, 2e-2, f"[{path}] {name}")


@pytest.mark.parametrize("name", ["c3_causal", "head", "pos_bidir", "pos_causal"])
def test_full_size_all_rows(name):
    # the L = 4096 workloads at their full shape (B4 H8), every output row
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype, norm_shells=w.norm_shells)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal, workers=O.default_workers())
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        if path == "generic" and w.causal:
            continue   # the generic kernels run this shape in test_generic_full_size_causal
        assert_parity(_run(dev, w.kind, w.causal, path), ref, 2e-2, f"[{path}] {name} all rows")


def test_generic_full_size_causal():
    # the float32-accumulating generic kernels on the causal full shape
    w = I.WORKLOADS["c3_causal"]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    rows = I.sample_rows(w.L, 256, seed=0)
    ref = O.favor_rows(q, k, v, W, w.kind, w.causal, rows)
    got = _run(dev, w.kind, w.causal, "generic")[..., rows, :]
    assert_parity(got, ref, 2e-2, "[generic] c3_causal sampled rows")


@pytest.mark.parametrize("name", ["c4_bidir", "c4_causal"])
def test_long_sequence_sampled_rows(name):
    # L = 32768: 256 sampled rows per head, each computed by the oracle
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype, norm_shells=w.norm_shells)
    rows = I.sample_rows(w.L, 256, seed=0)
    ref = O.favor_rows(q, k, v, W, w.kind, w.causal, rows)
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        got = _run(dev, w.kind, w.causal, path)[..., rows, :]
        assert_parity(got, ref, 2e-2, f"[{path}] {name} sampled rows")


@pytest.mark.parametrize("name", ["c4_bidir", "c4_causal"])
def test_long_sequence_all_rows(name):
    # L = 32768 at its full shape (B1 H8, key and query norms spread over
    # [0.5, 2]), every output row against the whole oracle: the bf16 split
    # partials (bidirectional, many token splits per head, summed by the
    # split-sum kernel) and the bf16 segment start states (causal, the
    # longest prefix scans) at the longest sequence
    w = I.WORKLOADS[name]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype, norm_shells=w.norm_shells)
    ref = O.favor_attention(q, k, v, W, w.kind, w.causal, workers=O.default_workers())
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal):
        assert_parity(_run(dev, w.kind, w.causal, path), ref, 2e-2, f"[{path}] {name} all rows")


@pytest.mark.parametrize("kind", ["trig", "positive"])
@pytest.mark.parametrize("BH", [(1, 4), (4, 8)], ids=["B1H4", "B4H8"])
def test_m512_long_all_rows(BH, kind):
    # the top of the pages' feature grid at a long sequence: L4096, m = 512,
    # bidirectional (MFMA readout in two feature passes).  B1 H4 runs
    # 4-wave readout blocks, B4 H8 the 8-wave ones.
    (B, H), L, d, m = BH, 4096, 64, 512
    assert F.favor_attention_resolve_path(B, H, L, d, m, "bf16", kind, False) == "mfma"
    dev, (q, k, v), W = problem(B, H, L, d, m, "bf16", seed=512)
    ref = O.favor_attention(q, k, v, W, kind, False, workers=O.default_workers())
    for path in _paths(B, H, L, d, m, "bf16", kind, False):
        assert_parity(_run(dev, kind, False, path), ref, 2e-2, f"[{path}] m512 {kind} {BH}")


def test_causal_matches_masked_form_c3_rows():
    # config 3 at its full shape (B4 H8 L4096) is also checked against the
    # explicitly masked quadratic form D^-1 (A . tril) V on 256 rows per
    # head: the chunk edges, segment edges and the ends are among them
    w = I.WORKLOADS["c3_causal"]
    dev, (q, k, v), W = problem(w.B, w.H, w.L, w.d, w.m, w.dtype)
    edges = [0, 1, 2, 3, 31, 32, 33, 63, 64, 511, 512, 1023, 1024, 2047, 2048, 4094, 4095]
    rows = np.unique(np.concatenate([edges, I.sample_rows(w.L, 256 - len(edges), seed=1)]))
    ref = O.favor_quadratic_rows(q, k, v, W, "trig", True, rows)
    for path in _paths(w.B, w.H, w.L, w.d, w.m, w.dtype, "trig", True):
        got = _run(dev, "trig", True, path)[..., rows, :]
        assert_parity(got, ref, 2e-2, f"[{path}] c3 masked form")


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
        assert_parity(from_device(out), ref, 2e-2, f"[{path}] garbage workspace")


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


def _big_key_problem(norm, heads_with_big=(0, 1)):
    # tokens 3, 100 and 257 of the given heads get keys of the given norm
    B, H, L, d, m = 1, 2, 300, 64, 256
    dev, (q, k, v), W = problem(B, H, L, d, m, "bf16", seed=11)
    r = np.random.default_rng(11)
    kb = k.copy()
    for t in (3, 100, 257):
        u = r.standard_normal((B, H, d))
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        for h in heads_with_big:
            kb[:, h, t] = norm * u[:, h]
    kst, k64 = I.to_storage(kb, "bf16")
    return dev, (q, k64, v), W, to_device(kst, "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("norm", [12.0, 30.0])
def test_trig_large_key_norms(norm, causal):
    # The trig key weight exp(|k~|^2 / 2) at d = 64: norm 30 gives
    # exp(56.25), below the float32 limit exp(88.7); such keys dominate the
    # rows that see them.  The bf16 projection's error grows with the key
    # norm (about 1.6e-2 per row at norm 30); the float32 kernels stay at
    # the bf16 output rounding.
    dev, (q, k64, v), W, kd = _big_key_problem(norm)
    ref = O.favor_attention(q, k64, v, W, "trig", causal)
    for path in _paths(1, 2, 300, 64, 256, "bf16", "trig", causal):
        got = F.favor_attention(dev[0], kd, dev[2], dev[3], kind="trig", causal=causal, path=path)
        torch.cuda.synchronize()
        assert_parity(from_device(got), ref, 2e-2, f"[{path}] key norm {norm} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_trig_key_weight_overflow(causal):
    # Beyond |k~|^2 / 2 = 88.7 (norm 37.7 at d = 64) the float32 key weight
    # overflows: the head with such keys has non-finite outputs (all of
    # them when bidirectional), and the other head is unaffected.
    dev, (q, k64, v), W, kd = _big_key_problem(40.0, heads_with_big=(0,))
    ref = O.favor_attention(q, k64, v, W, "trig", causal)
    for path in _paths(1, 2, 300, 64, 256, "bf16", "trig", causal):
        got = from_device(F.favor_attention(dev[0], kd, dev[2], dev[3], kind="trig", causal=causal,
                                            path=path))
        torch.cuda.synchronize()
        bad = ~np.isfinite(got[:, 0]).all(axis=-1)
        assert bad[:, 3:].all(), path        # every row that sees token 3
        if not causal:
            assert bad.all(), path
        assert_parity(got[:, 1:], ref[:, 1:], 2e-2, f"[{path}] head without large keys")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_more_heads_than_a_grid_dimension(dtype, d, causal):
    # B * H = 66 000 heads: beyond 65 535, the kernels that take the head
    # from the grid's y and z dimensions (and the MFMA ones, from a long x
    # dimension) must still reach every head.  Heads around the boundary
    # against the oracle, and bit for bit against the same heads run alone.
    B, H, L, m = 2, 33000, 5, 32
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=21)
    heads = [(0, 0), (1, 32534), (1, 32535), (1, 32999)]   # b * H + h = 0, 65534, 65535, 65999
    for path in _paths(B, H, L, d, m, dtype, "trig", causal):
        out = F.favor_attention(*dev, kind="trig", causal=causal, path=path)
        torch.cuda.synchronize()
        for b, h in heads:
            one = F.favor_attention(*(x[b:b + 1, h:h + 1].contiguous() for x in dev[:3]), dev[3],
                                    kind="trig", causal=causal, path=path)
            torch.cuda.synchronize()
            bits = torch.int16 if dtype == "bf16" else torch.int32
            assert torch.equal(out[b, h].view(bits), one[0, 0].view(bits)), (path, b, h)
            ref = O.favor_attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], W,
                                    "trig", causal)
            assert_parity(from_device(out[b:b + 1, h:h + 1]), ref, TOL[dtype], f"[{path}] head {b},{h}")


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
