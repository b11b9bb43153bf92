"""GPU checks of the masked-LM block helpers and the full block."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from linear_kernelized_attention_amd import inputs as I
from oracle import favor_oracle as O
from tests.gpu_util import from_device, to_device

pytestmark = pytest.mark.gpu


def test_embed_exact():
    b = I.block_inputs(B=2, L=300, E=512, seed=1)
    ids = torch.from_numpy(b.ids).cuda()
    table = to_device(b.embed, "bf16")
    x = F.favor_embed_bf16(ids, table)
    torch.cuda.synchronize()
    want = b.embed[b.ids]
    assert np.array_equal(x.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("M,N,K,ih,oh,seq", [
    (8192, 512, 512, 0, 8, 4096),     # Q/K/V projection, head-split output
    (8192, 512, 512, 8, 0, 4096),     # output projection, head-split input
    (8192, 1536, 512, 0, 0, 0),       # 128-column tiles
    (300, 96, 64, 0, 0, 0),           # ragged rows, N not a multiple of the tile
    (257, 200, 136, 0, 0, 0),         # K not a multiple of the 64-wide k step
    (1, 32, 32, 0, 0, 0),
    (1, 8, 8, 0, 0, 0),
])
def test_linear(M, N, K, ih, oh, seq):
    r = np.random.default_rng(M + N)
    X, X64 = I.to_storage(r.standard_normal((M, K)) * 0.5, "bf16")
    W, W64 = I.to_storage(r.standard_normal((K, N)) * 0.05, "bf16")
    if ih:
        # device X is head-split [B, ih, seq, K/ih]; logical X64 is [M, K]
        Bb = M // seq
        Xd = X.reshape(Bb, seq, ih, K // ih).transpose(0, 2, 1, 3).copy()
    else:
        Xd = X
    wt = F.favor_pack_weight_bf16(to_device(W, "bf16"))
    torch.cuda.synchronize()
    assert np.array_equal(wt.view(torch.int16).cpu().numpy().view(np.uint16), W.T)
    y = F.favor_linear_bf16(to_device(Xd, "bf16"), wt, M, N, K, ih, oh, seq)
    torch.cuda.synchronize()
    y = from_device(y)
    ref = X64 @ W64
    if oh:
        Bb = M // seq
        y = y.reshape(Bb, oh, seq, N // oh).transpose(0, 2, 1, 3).reshape(M, N)
    else:
        y = y.reshape(M, N)
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert err <= 4e-3, err


def test_performer_block_config5():
    cfg = I.BLOCK_WORKLOAD
    b = I.block_inputs(B=cfg["B"], L=cfg["L"], E=512, H=cfg["H"], seed=0)
    dr = I.omega_draws(cfg["m"], cfg["d"], seed=0)
    W = O.orthogonal_random_features(dr.gaussian, dr.radii, cfg["m"])
    ref = O.performer_block(b.ids, b.embed64, b.wq64, b.wk64, b.wv64, b.wo64, W, heads=cfg["H"],
                            kind="relu", workers=O.default_workers())
    omega = torch.from_numpy(F.favor_orf_omega(dr.gaussian, dr.radii, cfg["m"])).cuda()
    dev = [to_device(x, "bf16") for x in (b.embed, b.wq, b.wk, b.wv, b.wo)]
    weights = F.favor_block_weights(*dev[1:])
    ids = torch.from_numpy(b.ids).cuda()
    for path in ("generic", "auto"):
        y = F.favor_performer_block(ids, dev[0], weights, omega, heads=cfg["H"], kind="relu", path=path)
        torch.cuda.synchronize()
        y = from_device(y)
        for bi in range(cfg["B"]):
            err = np.linalg.norm(y[bi] - ref[bi]) / np.linalg.norm(ref[bi])
            print(f"[{path}] block batch {bi} rel={err:.3e}", flush=True)
            assert err <= 2e-2
        # no position signal: equal token ids give equal rows
        ids0 = b.ids[0]
        for t in (0, 5, 25):
            rows = y[0, ids0 == t]
            assert np.allclose(rows, rows[:1], atol=1e-6)


@pytest.mark.parametrize("M,N,K,heads,hd,seq,vocab", [
    (8192, 1536, 512, 8, 64, 4096, 26),   # the block's fused Q, K, V projection
    (300, 96, 64, 2, 16, 100, 7),         # ragged rows, 3 groups of 2 x 16
    (130, 40, 24, 0, 0, 0, 5),            # row-major output
])
def test_embed_linear(M, N, K, heads, hd, seq, vocab):
    r = np.random.default_rng(M + N + K)
    table, T64 = I.to_storage(r.standard_normal((vocab, K)) * 0.5, "bf16")
    W, W64 = I.to_storage(r.standard_normal((K, N)) * 0.05, "bf16")
    ids = r.integers(-2, vocab + 2, size=M).astype(np.int32)   # some ids out of range: zero rows
    wt = F.favor_pack_weight_bf16(to_device(W, "bf16"))
    y = F.favor_embed_linear_bf16(torch.from_numpy(ids).cuda(), to_device(table, "bf16"), wt, heads, hd, seq)
    torch.cuda.synchronize()
    y = from_device(y)
    X64 = np.where(((ids >= 0) & (ids < vocab))[:, None], T64[np.clip(ids, 0, vocab - 1)], 0.0)
    ref = X64 @ W64
    if heads:
        G = heads * hd
        Bb = M // seq
        # [N / G, B, heads, seq, hd] -> [M, N]
        y = y.reshape(N // G, Bb, heads, seq, hd).transpose(1, 3, 0, 2, 4).reshape(M, N)
    else:
        y = y.reshape(M, N)
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert err <= 4e-3, err
    # rows of out-of-range ids are exactly zero
    bad = (ids < 0) | (ids >= vocab)
    assert np.all(y[bad] == 0)
