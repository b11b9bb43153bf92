"""FAVOR attention throughput on one MI355X.

One step = one favor_attention call (scale, project, feature map,
key-side contraction, query readout, normalise and store) over the
headline workload: B=4, H=8, L=4096, d=64, m=256, bf16 inputs, trig
(sin/cos) features, bidirectional.  Inputs are synthetic (seeded
N(0,1) * d^-1/4) and resident in HBM before timing starts.

Prints one JSON line:
  value     = tokens x heads per second over the timed steps
  roofline  = the dominant kernel's algorithmic rate against the MI355X
              peak of the unit that bounds it, timed with HIP events on
              the launch stream inside this run
  cpu_baseline = the float64 CPU oracle on the same workload, host cores
  extra     = the other workloads (causal, long sequence, ReLU, the
              masked-LM block) timed the same way, for context

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-extra] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FAVOR attention (tokens x heads)/s at L=4096,d=64,m=256; % of MFMA/HBM roofline"
UNIT = "tokens*heads/s"

# MI355X published peaks
PEAK_BF16_MFMA_TFLOPS = 2516.6   # dense, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3
# untimed back-to-back calls before each other workload is timed, so that
# each is measured at the loaded clock and the last of them leaves the GPU
# there for the headline's warm-up and timed steps
EXTRA_SETTLE_S = 0.03

PROFILE_DIR = os.path.join(ROOT, "profiles")


def feature_width(m, kind):
    return 2 * m if kind == "trig" else m


def kernel_work(name: str, B, H, L, d, m, kind, esz=2):
    """(algorithmic flops, algorithmic HBM bytes) of one launch of a kernel.

    Per token-head (tok.h): projection 2dm flops per tensor, contraction
    2F(d+1) flops on the key side, readout 2F(d+1) flops on the query
    side; bytes: read Q, K, V and write out, d*esz each."""
    F = feature_width(m, kind)
    T = B * H * L
    proj = 2 * d * m
    con = 2 * F * (d + 1)
    if name.endswith("state") or "kv_state" in name:
        return T * (proj + con), T * 2 * d * esz
    if "readout" in name:
        if "causal" in name:
            return T * 2 * (proj + con), T * 4 * d * esz
        return T * (proj + con), T * 2 * d * esz
    return 0.0, 0.0


def path_total_work(B, H, L, d, m, kind, esz=2):
    F = feature_width(m, kind)
    T = B * H * L
    return T * (4 * d * m + 4 * F * (d + 1)), T * 4 * d * esz


def sources_sha256(names):
    """sha256 over the named kernel sources (csrc/), in order; None if any
    is missing."""
    h = hashlib.sha256()
    for n in names:
        p = os.path.join(ROOT, "linear_kernelized_attention_amd", "csrc", n)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest() if names else None


def load_traffic(kernel: str, workload: str = "head"):
    """HBM bytes per launch of a kernel (phase name) of a workload, from the
    committed rocprofv3 counter runs, if they were taken on the current
    kernel source; otherwise None."""
    fn = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(fn):
        return None
    try:
        rec = json.load(open(fn))
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    if not ent:
        return None
    if sources_sha256(ent.get("sources", [])) != ent.get("sources_sha256"):
        return None
    return float(ent["bytes_per_launch"])


def counter_bytes_per_call(workload: str, phases):
    """HBM bytes of one call from the counter runs (every phase of the call
    must have a current entry), or None."""
    total = 0.0
    for name, _ in phases:
        b = load_traffic(name, workload)
        if b is None:
            return None
        total += b
    return total


def upload_one(x, dtype):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def upload(ai, dtype):
    return [upload_one(x, dtype) for x in (ai.q, ai.k, ai.v)]


def time_calls(fn, steps, warmup, settle=0.0):
    """Seconds per call over `steps` timed calls after `warmup` untimed ones.
    With settle > 0, untimed calls first run back to back for that many
    seconds: the GPU raises its clocks over about 20 ms of continuous work
    (measured on the headline: 54 us per call at first, 44.5 us after
    400 calls) and drops them again when idle."""
    import torch
    if settle > 0:
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= settle:
                    break
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def prep_attention(F, I, w, path="auto"):
    """Uploads a workload's seeded inputs; returns run(steps, warmup) ->
    (seconds per favor_attention call, per-kernel phases, resolved path).
    Inputs are made before any timing starts, so that the timed blocks run
    back to back and the GPU does not idle (and drop its clocks) while the
    host draws the next workload's inputs."""
    import torch
    ai, dr = I.workload_inputs(w)
    q, k, v = upload(ai, w.dtype)
    omega = torch.from_numpy(F.favor_orf_omega(dr.gaussian, dr.radii, w.m)).cuda()
    out = torch.empty_like(q)
    need = F.favor_attention_workspace_bytes(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind, w.causal, path)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    fn = lambda: F.favor_attention(q, k, v, omega, kind=w.kind, causal=w.causal, path=path, out=out,
                                   workspace=ws)

    def run(steps, warmup, settle=0.0):
        sec = time_calls(fn, steps, warmup, settle)
        phases = F.favor_profile_attention(q, k, v, omega, kind=w.kind, causal=w.causal, path=path,
                                           iters=max(steps, 20), out=out, workspace=ws)
        resolved = F.favor_attention_resolve_path(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind,
                                                  w.causal, path)
        return sec, phases, resolved
    return run


def prep_block(F, I):
    """run(steps, warmup) -> seconds per masked-LM block call."""
    import torch
    cfg = I.BLOCK_WORKLOAD
    b = I.block_inputs(B=cfg["B"], L=cfg["L"], E=cfg["E"], H=cfg["H"], seed=0)
    dr = I.omega_draws(cfg["m"], cfg["d"], seed=0)
    omega = torch.from_numpy(F.favor_orf_omega(dr.gaussian, dr.radii, cfg["m"])).cuda()
    dev = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
           for x in (b.embed, b.wq, b.wk, b.wv, b.wo)]
    ids = torch.from_numpy(b.ids).cuda()
    weights = F.favor_block_weights(*dev[1:])   # packed once, as at model load
    fn = lambda: F.favor_performer_block(ids, dev[0], weights, omega, heads=cfg["H"], kind=cfg["kind"])
    return lambda steps, warmup, settle=0.0: time_calls(fn, steps, warmup, settle)


def prep_backward(F, I, w, saved=False):
    """run(steps, warmup) -> seconds per favor_attention_backward call on a workload's seeded
    inputs and a seeded N(0, 1) output gradient; with saved, the forward's
    (out, den) from favor_attention(..., den=True), made once before timing,
    is passed in (the training pattern)."""
    import torch
    ai, dr = I.workload_inputs(w)
    q, k, v = upload(ai, w.dtype)
    gs, _ = I.output_grads(w.B, w.H, w.L, w.d, w.dtype)
    g = upload_one(gs, w.dtype)
    omega = torch.from_numpy(F.favor_orf_omega(dr.gaussian, dr.radii, w.m)).cuda()
    need = F.favor_attention_backward_workspace_bytes(w.B, w.H, w.L, w.d, w.m, w.dtype, w.kind,
                                                      w.causal)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    sv = F.favor_attention(q, k, v, omega, kind=w.kind, causal=w.causal, den=True) if saved else None
    fn = lambda: F.favor_attention_backward(q, k, v, omega, g, kind=w.kind, causal=w.causal,
                                            workspace=ws, grads=grads, saved=sv)
    return lambda steps, warmup, settle=0.0: time_calls(fn, steps, warmup, settle)


def backward_work(B, H, L, d, m, kind):
    """Algorithmic flops of one backward call that recomputes the forward
    state: phi projections of q and k (4dm), S/z and num/den (4F(d+1)),
    dphi(q), R, dV and dphi(k) (8F(d+1)) and the projections' adjoints
    (4dm) per token-head."""
    F_ = feature_width(m, kind)
    return B * H * L * (8 * d * m + 12 * F_ * (d + 1))


def prep_random(F, shape, kind, causal):
    """run(steps, warmup) -> seconds per favor_attention call on random bf16 inputs of a shape
    (timing only: values N(0,1) d^-1/4 drawn on the device, Omega from the
    seeded orthogonal draw)."""
    import torch
    from linear_kernelized_attention_amd import inputs as I
    B, H, L, d, m = shape
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v = [(torch.randn(B, H, L, d, device="cuda", generator=g) * d ** -0.25).to(torch.bfloat16)
               for _ in range(3)]
    dr = I.omega_draws(m, d, seed=0)
    omega = torch.from_numpy(F.favor_orf_omega(dr.gaussian, dr.radii, m)).cuda()
    out = torch.empty_like(q)
    need = F.favor_attention_workspace_bytes(B, H, L, d, m, "bf16", kind, causal, "auto")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    fn = lambda: F.favor_attention(q, k, v, omega, kind=kind, causal=causal, out=out, workspace=ws)
    return lambda steps, warmup, settle=0.0: time_calls(fn, steps, warmup, settle)


def cpu_oracle_once(I, w):
    """tokens x heads per second of one pass of the float64 oracle on a
    workload (one worker per head, BLAS at 1 thread)."""
    from threadpoolctl import threadpool_limits

    from oracle import favor_oracle as O
    ai, dr = I.workload_inputs(w)
    W = O.orthogonal_random_features(dr.gaussian, dr.radii, w.m)
    workers = max(1, min(O.default_workers(), w.B * w.H))
    with threadpool_limits(1):
        t0 = time.perf_counter()
        O.favor_attention(ai.q64, ai.k64, ai.v64, W, w.kind, w.causal, workers=workers)
        el = time.perf_counter() - t0
    return w.tokens_x_heads / el


def blas_vendor() -> str:
    """The BLAS library numpy calls, as threadpoolctl reports it."""
    from threadpoolctl import threadpool_info
    libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
            if i.get("user_api") == "blas"]
    return ", ".join(sorted(set(libs))) or "unknown"


def cpu_baseline(I, w, min_seconds=10.0):
    """The float64 oracle, as it stands, on the whole headline workload
    (repeated until min_seconds of wall time), one worker thread per core."""
    from threadpoolctl import threadpool_limits

    from oracle import favor_oracle as O
    ai, dr = I.workload_inputs(w)
    W = O.orthogonal_random_features(dr.gaussian, dr.radii, w.m)
    cores = O.default_workers()
    workers = max(1, min(cores, w.B * w.H))
    reps = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while True:
            O.favor_attention(ai.q64, ai.k64, ai.v64, W, w.kind, w.causal, workers=workers)
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    el = time.perf_counter() - t0
    return {
        "value": reps * w.tokens_x_heads / el,
        "unit": UNIT,
        "cores": workers,
        "kind": "oracle",
        "blas": blas_vendor(),
        "sample": f"full workload B={w.B} H={w.H} L={w.L} d={w.d} m={w.m} {w.kind} "
                  f"{'causal' if w.causal else 'bidirectional'}, float64 numpy, {reps} pass(es) "
                  f"in {el:.1f} s, one worker per head, BLAS at 1 thread",
    }


def calibrate_copy(steps=5, mib=1024):
    """Plain device copies of known size (1 GiB read + 1 GiB written), for
    scaling the FETCH_SIZE/WRITE_SIZE counters: the runtime copy kernel and
    an elementwise kernel with 16-byte vector loads like this library's."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    for _ in range(steps):
        torch.add(x, 0.5, out=y)
    torch.cuda.synchronize()
    return mib * (1 << 20)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # enough warm-up for the GPU clocks to settle (a 20-call warm-up timed
    # about 13 % slow on the headline shape), then a long timed block
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--path", default="auto", choices=["auto", "generic", "mfma", "small"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    # instead of the throughput line: the estimator-quality sweep (error of
    # the GPU output against exact softmax over m and feature kinds)
    ap.add_argument("--estimator-sweep", action="store_true")
    # instead of the throughput line: time one other workload alone (a
    # forward workload name, "bwd_<workload>" for the backward pass,
    # "bwds_<workload>" for it with the saved forward, or "block"), e.g. to
    # profile its kernels
    ap.add_argument("--only", default=None)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_kernelized_attention_amd as F
    from linear_kernelized_attention_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.estimator_sweep:
        from linear_kernelized_attention_amd import sweep
        print(json.dumps(sweep.run()), flush=True)
        return
    if args.calibrate_copy:
        nbytes = calibrate_copy()
        print(json.dumps({"copy_calibration_bytes_read": nbytes}), flush=True)
    if args.only:
        key = args.only
        if key == "block":
            sec = prep_block(F, I)(args.steps, args.warmup)
            rec = {"only": key, "us_per_call": sec * 1e6}
        elif key.startswith("bwd_") or key.startswith("bwds_"):
            saved = key.startswith("bwds_")
            wk = I.WORKLOADS[key.split("_", 1)[1]]
            sec = prep_backward(F, I, wk, saved)(args.steps, args.warmup)
            rec = {"only": key, "us_per_call": sec * 1e6,
                   "algorithmic_tflops": backward_work(wk.B, wk.H, wk.L, wk.d, wk.m, wk.kind) / sec / 1e12}
        else:
            wk = I.WORKLOADS[key]
            sec, ph, rp = prep_attention(F, I, wk, args.path)(args.steps, args.warmup)
            rec = {"only": key, "us_per_call": sec * 1e6, "path": rp, "phases_ms": {n: t for n, t in ph}}
        print(json.dumps(rec), flush=True)
        return
    # Every workload's inputs are drawn and uploaded before the first timed
    # block; the other workloads then run first, back to back, for the
    # record's "extra" field, which leaves the GPU at its steady-state
    # clocks for the headline's warm-up and timed steps that follow.
    w = I.WORKLOADS["head"]
    head_run = prep_attention(F, I, w, args.path)
    extra = None
    if not args.no_extra:
        fwd_keys = ("c3_causal", "c2_trig", "c2_relu", "c4_bidir", "c4_causal", "c1", "pos_bidir",
                    "pos_causal")
        bwd_keys = (("head", False), ("c3_causal", False), ("c2_trig", False), ("head", True),
                    ("c3_causal", True))
        cfg = I.BLOCK_WORKLOAD
        fwd_runs = {key: prep_attention(F, I, I.WORKLOADS[key], "auto") for key in fwd_keys}
        block_run = prep_block(F, I)
        block_favor_run = prep_random(F, (cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["m"]),
                                      cfg["kind"], False)
        bwd_runs = {(key, saved): prep_backward(F, I, I.WORKLOADS[key], saved) for key, saved in bwd_keys}
        sweep_runs = {Bs: prep_random(F, (Bs, w.H, w.L, w.d, w.m), w.kind, w.causal) for Bs in (8, 16, 32)}
        torch.cuda.synchronize()

        extra = {}
        steps = max(10, args.steps // 4)
        settle = EXTRA_SETTLE_S
        for key in fwd_keys:
            wk = I.WORKLOADS[key]
            s, ph, rp = fwd_runs[key](steps, max(3, args.warmup // 4), settle)
            fl, by = path_total_work(wk.B, wk.H, wk.L, wk.d, wk.m, wk.kind, 4 if wk.dtype == "f32" else 2)
            extra[key] = {"us_per_call": s * 1e6, "tokens_x_heads_per_s": wk.tokens_x_heads / s,
                          "path": rp, "mfma_frac": fl / s / 1e12 / PEAK_BF16_MFMA_TFLOPS,
                          "hbm_frac": by / s / 1e9 / PEAK_HBM_GBS,
                          "phases_ms": {n: t for n, t in ph}}
            # HBM bytes actually moved (FETCH_SIZE + WRITE_SIZE counters),
            # the state streaming of the causal path included
            cb = counter_bytes_per_call(key, ph)
            if cb is not None:
                extra[key]["hbm_counter_bytes_per_call"] = cb
                extra[key]["hbm_counter_frac"] = cb / s / 1e9 / PEAK_HBM_GBS
        sb = block_run(steps, 3, settle)
        sf = block_favor_run(steps, 3, settle)
        extra["c5_block"] = {"us_per_call": sb * 1e6, "tokens_per_s": cfg["B"] * cfg["L"] / sb,
                             "favor_us_per_call": sf * 1e6}
        # backward pass on the headline, causal and B8 H8 L1024 shapes, and
        # (bwds_) with the forward's saved output and row normalisers
        for key, saved in bwd_keys:
            wk = I.WORKLOADS[key]
            sbw = bwd_runs[(key, saved)](steps, max(3, args.warmup // 4), settle)
            fl = backward_work(wk.B, wk.H, wk.L, wk.d, wk.m, wk.kind)
            rp = F.favor_attention_backward_resolve_path(wk.B, wk.H, wk.L, wk.d, wk.m, wk.dtype,
                                                         wk.kind, wk.causal)
            peak = PEAK_BF16_MFMA_TFLOPS if rp == "mfma" else PEAK_FP32_VALU_TFLOPS
            extra[f"{'bwds' if saved else 'bwd'}_{key}"] = {"us_per_call": sbw * 1e6, "tokens_x_heads_per_s": wk.tokens_x_heads / sbw,
                                   "path": rp, "algorithmic_tflops": fl / sbw / 1e12,
                                   "peak_frac": fl / sbw / 1e12 / peak,
                                   "peak": "bf16 MFMA" if rp == "mfma" else "fp32 VALU"}
        # saturation: the headline shape at larger batch (timing on random inputs)
        sweep = {}
        for Bs, run in sweep_runs.items():
            ss = run(steps, 3, settle)
            fl, _ = path_total_work(Bs, w.H, w.L, w.d, w.m, w.kind)
            sweep[f"B{Bs}"] = {"us_per_call": ss * 1e6, "tokens_x_heads_per_s": Bs * w.H * w.L / ss,
                               "mfma_frac": fl / ss / 1e12 / PEAK_BF16_MFMA_TFLOPS}
        extra["head_sweep"] = sweep

    sec, phases, resolved = head_run(args.steps, args.warmup)
    value = w.tokens_x_heads / sec

    # dominant kernel: the longest phase of one call
    name, ms = max(phases, key=lambda p: p[1])
    flops, nbytes = kernel_work(name, w.B, w.H, w.L, w.d, w.m, w.kind)
    mfma = resolved == "mfma"
    if mfma:
        achieved = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_MFMA_TFLOPS}
    else:
        achieved = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS}
    roof["traffic"] = load_traffic(name)
    roof["kernel"] = name
    roof["kernel_ms"] = ms
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = nbytes
    tot_flops, tot_bytes = path_total_work(w.B, w.H, w.L, w.d, w.m, w.kind)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1)*d^-1/4 Q,K,V; ORF Omega (4 blocks of 64x64)",
        "config": {"workload": "favor_attention bidirectional trig", "B": w.B, "H": w.H, "L": w.L,
                   "d": w.d, "m": w.m, "kind": w.kind, "causal": w.causal, "path": resolved},
        "roofline": roof,
        "step_mfma_frac": tot_flops / sec / 1e12 / PEAK_BF16_MFMA_TFLOPS,
        "step_hbm_frac": tot_bytes / sec / 1e9 / PEAK_HBM_GBS,
        "phases_ms": {n: t for n, t in phases},
    }

    if extra is not None:
        rec["extra"] = extra

    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(I, w)
        if "extra" in rec:
            for key in ("c1", "c2_trig", "c2_relu", "c3_causal", "c4_bidir", "c4_causal", "pos_bidir", "pos_causal"):
                rec["extra"][key]["cpu_oracle_tokens_x_heads_per_s"] = cpu_oracle_once(I, I.WORKLOADS[key])
    else:
        rec["cpu_baseline"] = None

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
