"""favor_attention_noalloc (the entry point that allocates nothing; its
scratch is a fixed per-device array inside the library) against
favor_attention with a caller-supplied workspace, through the C ABI: two
calls in a row on each path, the second on a smaller input, each compared
with the workspace entry point's output bit for bit (same kernels, fixed
reduction order) and with the oracle within the parity bar."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from oracle import favor_oracle as O
from tests.gpu_util import TOL, assert_parity, from_device, problem

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, L, d, m, dtype, kind, causal): the first call of each pair is
    # the larger input
    ((4, 8, 4096, 64, 256, "bf16", "trig", False), (1, 3, 257, 64, 256, "bf16", "trig", False)),
    ((4, 8, 4096, 64, 256, "bf16", "trig", True), (1, 2, 300, 64, 256, "bf16", "trig", True)),
    ((2, 4, 1000, 64, 128, "bf16", "positive", True), (1, 1, 33, 64, 128, "bf16", "positive", True)),
    ((1, 2, 512, 16, 64, "f32", "trig", False), (1, 1, 100, 16, 64, "f32", "trig", False)),
]


def _noalloc_vs_workspace(shape, seed):
    B, H, L, d, m, dtype, kind, causal = shape
    dev, (q, k, v), W = problem(B, H, L, d, m, dtype, seed=seed)
    ref_ws = F.favor_attention(*dev, kind=kind, causal=causal)
    got = F.favor_attention_noalloc(*dev, kind=kind, causal=causal)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(got.view(bits), ref_ws.view(bits)), shape
    ref = O.favor_attention(q, k, v, W, kind, causal, workers=O.default_workers())
    assert_parity(from_device(got), ref, TOL[dtype], f"noalloc {shape}")


@pytest.mark.parametrize("pair", CASES, ids=[f"{c[0][6]}_{'causal' if c[0][7] else 'bidir'}_{c[0][5]}" for c in CASES])
def test_noalloc_matches_workspace_entry_point(pair):
    big, small = pair
    print(f"noalloc case {big} then {small}", flush=True)
    _noalloc_vs_workspace(big, seed=21)
    _noalloc_vs_workspace(small, seed=22)
