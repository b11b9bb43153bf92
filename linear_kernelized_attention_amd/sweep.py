"""Estimator-quality sweep: how far FAVOR attention, computed on the GPU,
is from exact softmax attention as the number of random features m and
the kind of random features (orthogonal or i.i.d.) change.

The pages grid-search m over {64, 128, 256, 512} and report that too few
features flatten the attention ("Masked Language Modeling for Proteins
..." summary pages, 实验设计 / Results; FAVOR+ blog page, section
核心机制：FAVOR+), and that orthogonal features lower the estimator's
variance.  The sweep measures both on the device: for each setting it
runs favor_attention on seeded synthetic inputs and compares sampled
output rows with softmax(q k^T / sqrt(d)) v, evaluated here in float64
from the stored bf16 values (a comparison target, not part of the path).

Usage: python -m linear_kernelized_attention_amd.sweep [--L 4096] [--H 8]
prints one JSON object; bench.py --estimator-sweep runs the same sweep.
"""
from __future__ import annotations

import argparse
import json

import numpy as np

from . import inputs as I

# Input scales, as multiples of the workloads' draw N(0, 1) * d^-1/4:
# "x1" (q.k / sqrt(d) of standard deviation about d^-1/2: nearly uniform
# attention, |x~|^2 / 2 about 1/2) and "x1.5" (standard deviation about
# 0.28, |x~|^2 / 2 about 1.1).  The estimators' variance grows like
# e^{|x~|^2} (trig weights e^{|x~|^2/2}), so at d = 64 and m <= 512 the
# error is already large at x1.5 and runs away beyond x2.
SCALES = {"x1": 1.0, "x1.5": 1.5}


def _inputs(H: int, L: int, d: int, scale: str, seed: int):
    a = I.attention_inputs(1, H, L, d, "bf16", seed=seed)
    f = SCALES[scale]
    if f == 1.0:
        return a
    qs, q64 = I.to_storage(a.q64 * f, "bf16")
    ks, k64 = I.to_storage(a.k64 * f, "bf16")
    return I.AttentionInputs(1, H, L, d, "bf16", qs, ks, a.v, q64, k64, a.v64)


def softmax_rows(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Exact bidirectional softmax attention at the given rows of each head:
    [H, len(rows), d] from [H, L, d] float64 arrays."""
    d = q64.shape[-1]
    out = np.empty((q64.shape[0], len(rows), d))
    for h in range(q64.shape[0]):
        s = q64[h, rows] @ k64[h].T / np.sqrt(d)
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        out[h] = (w @ v64[h]) / w.sum(axis=1, keepdims=True)
    return out


def run(L: int = 4096, H: int = 8, d: int = 64, ms=(64, 128, 256, 512), kinds=("trig", "positive"),
        scales=tuple(SCALES), seeds=(0, 1, 2, 3), n_rows: int = 256, input_seed: int = 0) -> dict:
    """Relative Frobenius error of the GPU output against softmax attention
    on n_rows sampled rows per head, for every (scale, kind, m, features)
    over Omega seeds; returns {"rows": [...], ...}."""
    import torch
    from . import _lib as F

    rows = np.sort(I.rng(input_seed, "rows").choice(L, size=min(n_rows, L), replace=False))
    res = []
    for scale in scales:
        a = _inputs(H, L, d, scale, input_seed)
        ref = softmax_rows(a.q64[0], a.k64[0], a.v64[0], rows)
        dev = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
               for x in (a.q, a.k, a.v)]
        for kind in kinds:
            for m in ms:
                for feat in ("orf", "iid"):
                    errs = []
                    path = None
                    for s in seeds:
                        if feat == "orf":
                            dr = I.omega_draws(m, d, seed=1000 + s)
                            om = F.favor_orf_omega(dr.gaussian, dr.radii, m)
                        else:
                            om = I.iid_gaussian_omega(m, d, seed=1000 + s).astype(np.float32)
                        omega = torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda()
                        out = F.favor_attention(*dev, omega, kind=kind, causal=False)
                        path = F.favor_attention_resolve_path(1, H, L, d, m, "bf16", kind, False)
                        torch.cuda.synchronize()
                        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
                        got = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0][:, rows]
                        e = [np.linalg.norm(got[h] - ref[h]) / np.linalg.norm(ref[h]) for h in range(H)]
                        errs.append(float(np.mean(e)))
                    res.append({"scale": scale, "kind": kind, "m": m, "features": feat, "path": path,
                                "rel_err_mean": float(np.mean(errs)), "rel_err_std": float(np.std(errs)),
                                "seeds": len(seeds)})
    return {"workload": f"B1 H{H} L{L} d{d} bf16 bidirectional", "rows_per_head": int(len(rows)),
            "metric": "relative Frobenius error vs exact softmax attention, mean over heads",
            "rows": res}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--L", type=int, default=4096)
    ap.add_argument("--H", type=int, default=8)
    args = ap.parse_args()
    print(json.dumps(run(L=args.L, H=args.H)), flush=True)


if __name__ == "__main__":
    main()
