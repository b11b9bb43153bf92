"""The forward under HIP graph capture and on a non-default stream.

`favor_attention` (with a caller workspace) and `favor_attention_noalloc`
(the library's fixed scratch) enqueue only kernel launches on the caller's
stream, so a captured call replays like the eager one: each replay below
runs on new inputs copied into the captured tensors between replays, and
must match an eager call on the same inputs bit for bit."""
import numpy as np
import pytest
import torch

import linear_kernelized_attention_amd as F
from tests.gpu_util import problem

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, L, d, m, dtype, kind, causal): MFMA bidirectional and causal,
    # the small float32 path
    (1, 4, 1000, 64, 256, "bf16", "trig", False),
    (1, 4, 1000, 64, 256, "bf16", "positive", True),
    (1, 2, 300, 16, 64, "f32", "trig", False),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[6]}_{'causal' if c[7] else 'bidir'}_{c[5]}" for c in CASES])
def test_captured_forward_replays(case, entry):
    B, H, L, d, m, dtype, kind, causal = case
    dev, _, _ = problem(B, H, L, d, m, dtype, seed=31)
    q, k, v, w = (x.clone() for x in dev)
    out = torch.empty_like(q)
    if entry == "workspace":
        need = F.favor_attention_workspace_bytes(B, H, L, d, m, dtype, kind, causal)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        fn = lambda: F.favor_attention(q, k, v, w, kind=kind, causal=causal, out=out, workspace=ws)
    else:
        fn = lambda: F.favor_attention_noalloc(q, k, v, w, kind=kind, causal=causal, out=out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the default stream
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    for rep in range(4):
        new, _, _ = problem(B, H, L, d, m, dtype, seed=100 + rep)
        for dst, src in zip((q, k, v), new[:3]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = F.favor_attention(q, k, v, w, kind=kind, causal=causal)
        torch.cuda.synchronize()
        assert torch.isfinite(eager.float()).all()
        assert torch.equal(_bits(out), _bits(eager)), (entry, case, rep)
