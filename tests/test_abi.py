"""C-ABI checks that need no GPU: the library loads, exports every function
include/favor.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import _lib as B
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "favor.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(favor_\w+)\s*\(", text)))


def test_every_declared_symbol_exported():
    lib = F.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_library_resolves_every_symbol_at_load():
    # immediate binding: an internal function declared but left undefined
    # would otherwise surface only at its first call
    ctypes.CDLL(B.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_single_hip_runtime():
    F.lib()
    assert len(F.loaded_hip_runtimes()) <= 1


def test_version_and_status_strings():
    lib = F.lib()
    assert lib.favor_version() > 0
    for s in (0, -1, -2, -3, -4, -5):
        assert F.status_string(s) and F.status_string(s) != "unknown status"
    assert F.status_string(7) == "unknown status"


# Fake, never-dereferenced addresses: every call below must return before
# touching memory or launching anything.
QA, KA, VA, WA, OA, WS = (0x100000 * i for i in range(1, 7))


def call(q=QA, k=KA, v=VA, w=WA, o=OA, B_=2, H=2, L=64, d=64, m=256, dt=1, kind=0, causal=0,
         ws=WS, wsb=1 << 30, path=0):
    return F.lib().favor_attention_ex(q, k, v, w, o, B_, H, L, d, m, dt, kind, causal, ws, wsb, None,
                                      path)


def test_invalid_arguments():
    assert call(q=0) == B.FAVOR_ERR_INVALID_ARG
    assert call(o=0) == B.FAVOR_ERR_INVALID_ARG
    assert call(w=0) == B.FAVOR_ERR_INVALID_ARG
    assert call(B_=-1) == B.FAVOR_ERR_INVALID_ARG
    assert call(d=0) == B.FAVOR_ERR_INVALID_ARG
    assert call(m=0) == B.FAVOR_ERR_INVALID_ARG
    assert call(dt=2) == B.FAVOR_ERR_INVALID_ARG
    assert call(kind=5) == B.FAVOR_ERR_INVALID_ARG
    assert call(causal=2) == B.FAVOR_ERR_INVALID_ARG
    assert call(path=9) == B.FAVOR_ERR_INVALID_ARG


def test_misaligned_pointers():
    # every device pointer must be 16-byte aligned
    assert call(q=QA + 2) == B.FAVOR_ERR_INVALID_ARG
    assert call(k=KA + 8) == B.FAVOR_ERR_INVALID_ARG
    assert call(v=VA + 4) == B.FAVOR_ERR_INVALID_ARG
    assert call(w=WA + 4) == B.FAVOR_ERR_INVALID_ARG
    assert call(o=OA + 2) == B.FAVOR_ERR_INVALID_ARG
    assert call(ws=WS + 8) == B.FAVOR_ERR_INVALID_ARG


def test_empty_problem_is_noop():
    for kw in (dict(L=0), dict(B_=0), dict(H=0)):
        assert call(q=0, k=0, v=0, w=0, o=0, ws=0, wsb=0, **kw) == B.FAVOR_OK


def test_unsupported():
    assert call(d=128) == B.FAVOR_ERR_UNSUPPORTED
    assert call(m=4096) == B.FAVOR_ERR_UNSUPPORTED
    # the MFMA family needs bf16 and d = 64
    assert call(dt=0, d=16, m=64, path=2) == B.FAVOR_ERR_UNSUPPORTED


def test_workspace_checks():
    need = F.favor_attention_workspace_bytes(2, 2, 64, 64, 256, "bf16", "trig", False)
    assert need > 0
    assert call(ws=0) == B.FAVOR_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.FAVOR_ERR_WORKSPACE


def test_alias_checks():
    assert call(o=QA) == B.FAVOR_ERR_ALIAS
    assert call(o=VA + 64) == B.FAVOR_ERR_ALIAS
    assert call(ws=OA) == B.FAVOR_ERR_ALIAS


def test_workspace_sizes_monotone():
    a = F.favor_attention_workspace_bytes(1, 8, 4096, 64, 256, "bf16", "trig", True)
    b = F.favor_attention_workspace_bytes(1, 8, 32768, 64, 256, "bf16", "trig", True)
    assert 0 < a <= b
    assert F.favor_attention_workspace_bytes(1, 1, 512, 16, 64, "f32", "trig", False) > 0
    assert F.favor_attention_workspace_bytes(1, 1, 0, 16, 64, "f32", "trig", False) == 0


def test_resolve_path():
    # the small float32 workload runs on the small path (its one-launch
    # kernel at this size); the generic kernels take it when asked, MFMA
    # cannot
    R = F.favor_attention_resolve_path
    assert R(1, 1, 512, 16, 64, "f32", "trig", False) == "small"
    assert R(1, 1, 512, 16, 64, "f32", "trig", False, "generic") == "generic"
    assert R(1, 1, 512, 16, 64, "f32", "trig", False, "small") == "small"
    with pytest.raises(F.FavorError):
        R(1, 1, 512, 16, 64, "f32", "trig", False, "mfma")
    # the small path: bidirectional, d <= 32, m <= 128, L <= 1024
    for args in ((1, 1, 512, 16, 64, "f32", "trig", True), (1, 1, 512, 64, 64, "f32", "trig", False),
                 (1, 1, 512, 16, 256, "f32", "trig", False), (1, 1, 2048, 16, 64, "f32", "trig", False)):
        assert R(*args) == "generic"
        with pytest.raises(F.FavorError):
            R(*args, "small")
    assert R(2, 4, 1024, 32, 128, "bf16", "relu", False) == "small"
    # no backward kernels in the small family
    assert F.favor_attention_backward_workspace_bytes(1, 1, 512, 16, 64, "f32", "trig", False, "small") == 0


@pytest.mark.parametrize("kind", ["trig", "relu", "positive"])
def test_resolve_path_feature_counts(kind):
    # MFMA takes m a multiple of 32 up to 256 in both directions, and m = 512
    # for the bidirectional forward only; everything else is generic
    R, RB = F.favor_attention_resolve_path, F.favor_attention_backward_resolve_path
    for m in (32, 96, 256):
        for causal in (False, True):
            assert R(1, 4, 4096, 64, m, "bf16", kind, causal) == "mfma"
    assert R(1, 4, 4096, 64, 512, "bf16", kind, False) == "mfma"
    assert R(1, 4, 4096, 64, 512, "bf16", kind, True) == "generic"
    assert RB(1, 4, 4096, 64, 512, "bf16", kind, False) == "generic"
    assert RB(1, 4, 4096, 64, 512, "bf16", kind, True) == "generic"
    for m in (288, 384, 1024):
        assert R(1, 4, 4096, 64, m, "bf16", kind, False) == "generic"
    with pytest.raises(F.FavorError):
        R(1, 4, 4096, 64, 512, "bf16", kind, True, "mfma")


def test_linear_and_embed_argument_checks():
    lib = F.lib()
    assert lib.favor_linear_bf16(QA, KA, OA, 0, 64, 64, 0, 0, 0, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_linear_bf16(QA, KA, OA, 64, 44, 64, 0, 0, 0, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_linear_bf16(QA, KA, OA, 64, 64, 64, 0, 3, 64, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_linear_bf16(QA, KA, QA, 64, 64, 64, 0, 0, 0, None) == B.FAVOR_ERR_ALIAS
    assert lib.favor_linear_bf16(QA, KA, OA, 100, 64, 64, 0, 2, 64, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_embed_bf16(0, KA, OA, 10, 26, 512, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_embed_bf16(0, 0, 0, 0, 26, 512, None) == B.FAVOR_OK
    assert lib.favor_embed_bf16(QA, KA, OA, 10, 26, 12, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_embed_bf16(QA, KA + 2, OA, 10, 26, 512, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_linear_bf16(QA + 2, KA, OA, 64, 64, 64, 0, 0, 0, None) == B.FAVOR_ERR_INVALID_ARG
    # weight packing
    assert lib.favor_pack_weight_bf16(QA, OA, 0, 64, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_pack_weight_bf16(QA, 0, 64, 64, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_pack_weight_bf16(QA, QA + 64, 64, 64, None) == B.FAVOR_ERR_ALIAS
    # fused gather + projection: ids, table, vocab, Wt, Y, M, N, K, heads, head_dim, seq
    ids = QA + (1 << 26)
    assert lib.favor_embed_linear_bf16(0, KA, 26, VA, OA, 64, 192, 64, 0, 0, 0, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_embed_linear_bf16(ids, KA, 0, VA, OA, 64, 192, 64, 0, 0, 0, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_embed_linear_bf16(ids, KA, 26, VA, OA, 64, 196, 64, 0, 0, 0, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_embed_linear_bf16(ids, KA, 26, VA, OA, 64, 192, 64, 2, 36, 32, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_embed_linear_bf16(ids, KA, 26, VA, OA, 64, 200, 64, 2, 32, 32, None) == B.FAVOR_ERR_UNSUPPORTED
    assert lib.favor_embed_linear_bf16(ids, KA, 26, VA, OA, 60, 192, 64, 2, 32, 32, None) == B.FAVOR_ERR_INVALID_ARG
    assert lib.favor_embed_linear_bf16(ids, KA, 26, VA, KA, 64, 192, 64, 0, 0, 0, None) == B.FAVOR_ERR_ALIAS


@pytest.mark.parametrize("m,d", [(64, 16), (256, 64), (40, 16)])
def test_host_orf_matches_oracle(m, d):
    # the library's host ORF (float64 Gram-Schmidt, float32 output) against
    # the oracle's, from the same raw draws
    dr = I.omega_draws(m, d, seed=0)
    ours = F.favor_orf_omega(dr.gaussian, dr.radii, m)
    ref = O.orthogonal_random_features(dr.gaussian, dr.radii, m)
    assert ours.dtype == np.float32 and ours.shape == (m, d)
    assert np.abs(ours - ref).max() <= 4e-7 * np.abs(ref).max()


def test_host_orf_rejects_degenerate_block():
    g = np.zeros((1, 4, 4))
    with pytest.raises(F.FavorError):
        F.favor_orf_omega(g, np.ones(4), 4)


# ------------------------------------------------------------- backward
GA, DQA, DKA, DVA = (0x100000 * i for i in range(7, 11))


def bcall(q=QA, k=KA, v=VA, w=WA, g=GA, dq=DQA, dk=DKA, dv=DVA, B_=2, H=2, L=64, d=64, m=256,
          dt=1, kind=0, causal=0, ws=WS, wsb=1 << 40):
    return F.lib().favor_attention_backward(q, k, v, w, g, dq, dk, dv, B_, H, L, d, m, dt, kind,
                                            causal, ws, wsb, None)


def test_backward_argument_checks():
    assert bcall(g=0) == B.FAVOR_ERR_INVALID_ARG
    assert bcall(dk=0) == B.FAVOR_ERR_INVALID_ARG
    assert bcall(kind=7) == B.FAVOR_ERR_INVALID_ARG
    assert bcall(dv=DVA + 8) == B.FAVOR_ERR_INVALID_ARG      # misaligned
    assert bcall(d=128) == B.FAVOR_ERR_UNSUPPORTED
    assert bcall(ws=0) == B.FAVOR_ERR_WORKSPACE
    need = F.favor_attention_backward_workspace_bytes(2, 2, 64, 64, 256, "bf16", "trig", False)
    assert need > 0 and bcall(wsb=need - 1) == B.FAVOR_ERR_WORKSPACE
    assert bcall(q=0, k=0, v=0, w=0, g=0, dq=0, dk=0, dv=0, ws=0, wsb=0, L=0) == B.FAVOR_OK


def test_backward_alias_checks():
    assert bcall(dq=QA) == B.FAVOR_ERR_ALIAS          # output over an input
    assert bcall(dk=GA + 64) == B.FAVOR_ERR_ALIAS     # output over dOut
    assert bcall(dv=DKA) == B.FAVOR_ERR_ALIAS         # outputs overlap each other
    assert bcall(ws=DQA) == B.FAVOR_ERR_ALIAS         # workspace over an output


# saved-forward entry points: den [B, H, L] float32 and the saved output;
# the backward's workspace sits above every other fake buffer
DENA, SOA, BWS = 0x100000 * 11, 0x100000 * 12, 0x100000 * 64


def tcall(den=DENA, o=OA, q=QA, ws=WS, L=64, path=0):
    return F.lib().favor_attention_train(q, KA, VA, WA, o, den, 2, 2, L, 64, 256, 1, 0, 0, ws,
                                         1 << 30, None, path)


def scall(out=SOA, den=DENA, dq=DQA, ws=BWS, L=64):
    return F.lib().favor_attention_backward_saved(QA, KA, VA, WA, out, den, GA, dq, DKA, DVA, 2, 2,
                                                  L, 64, 256, 1, 0, 0, ws, 1 << 40, None, 0)


def test_saved_forward_argument_checks():
    assert tcall(den=0) == B.FAVOR_ERR_INVALID_ARG
    assert tcall(den=DENA + 2) == B.FAVOR_ERR_INVALID_ARG     # misaligned
    assert tcall(den=OA + 16) == B.FAVOR_ERR_ALIAS            # over the output
    assert tcall(den=QA) == B.FAVOR_ERR_ALIAS                 # over an input
    assert tcall(den=WS + 64) == B.FAVOR_ERR_ALIAS            # over the workspace
    assert tcall(path=9) == B.FAVOR_ERR_INVALID_ARG
    assert tcall(den=0, o=0, q=0, ws=0, L=0) == B.FAVOR_OK     # empty: nothing touched
    assert scall(out=0) == B.FAVOR_ERR_INVALID_ARG
    assert scall(den=0) == B.FAVOR_ERR_INVALID_ARG
    assert scall(out=SOA + 8) == B.FAVOR_ERR_INVALID_ARG      # misaligned
    assert scall(dq=SOA) == B.FAVOR_ERR_ALIAS                 # gradient over the saved output
    assert scall(dq=DENA) == B.FAVOR_ERR_ALIAS                # gradient over den
    assert scall(ws=DENA) == B.FAVOR_ERR_ALIAS                # workspace over den
    assert scall(L=0, out=0, den=0) == B.FAVOR_OK


def test_backward_workspace_covers_forward_state():
    shape = (1, 8, 4096, 64, 256, "bf16", "trig")
    for causal in (False, True):
        fwd = F.favor_attention_workspace_bytes(*shape, causal, "generic")
        bwd = F.favor_attention_backward_workspace_bytes(*shape, causal, "generic")
        assert bwd > fwd
    for causal in (False, True):
        assert (F.favor_attention_backward_workspace_bytes(*shape, causal, "mfma")
                > F.favor_attention_workspace_bytes(*shape, causal, "mfma"))
        assert F.favor_attention_backward_resolve_path(1, 8, 4096, 64, 256, "bf16", "trig", causal) == "mfma"
    # outside the MFMA family (float32, or d != 64) the generic kernels run
    assert F.favor_attention_backward_workspace_bytes(1, 8, 4096, 64, 256, "f32", "trig", True, "mfma") == 0
    assert F.favor_attention_backward_resolve_path(1, 8, 4096, 32, 256, "bf16", "trig", True) == "generic"


def noalloc(q=QA, k=KA, v=VA, w=WA, o=OA, B_=2, H=2, L=64, d=64, m=256, dt=1, kind=0, causal=0,
            path=0):
    return F.lib().favor_attention_noalloc(q, k, v, w, o, B_, H, L, d, m, dt, kind, causal, None,
                                           path)


def test_noalloc_host_checks():
    # the entry point without a workspace argument checks its arguments and
    # its scratch limit before it touches a device
    assert noalloc(q=0) == B.FAVOR_ERR_INVALID_ARG
    assert noalloc(dt=3) == B.FAVOR_ERR_INVALID_ARG
    assert noalloc(path=7) == B.FAVOR_ERR_INVALID_ARG
    assert noalloc(d=128) == B.FAVOR_ERR_UNSUPPORTED
    for kw in (dict(L=0), dict(B_=0)):
        assert noalloc(q=0, k=0, v=0, w=0, o=0, **kw) == B.FAVOR_OK
    # beyond FAVOR_NOALLOC_SCRATCH_BYTES (64 MiB): rejected, nothing enqueued
    big = dict(B_=64, H=8, L=32768, causal=1)
    assert F.favor_attention_workspace_bytes(64, 8, 32768, 64, 256, "bf16", "trig", True) > 64 << 20
    assert noalloc(**big) == B.FAVOR_ERR_WORKSPACE
