"""Seeded synthetic inputs for FAVOR attention workloads.

This module holds random draws and storage-format conversions only: it
computes no part of the attention method itself.  Both the CPU oracle
(under ``oracle/``) and the GPU path receive their inputs from here, so
the two sides see bit-identical Q, K, V and the same raw random draws
from which each side builds its own orthogonal random-feature matrix.

Generator: numpy PCG64 via ``default_rng([seed, stream])``, one stream
per tensor (see ``STREAM``).  Values are drawn in float64, scaled, rounded
to float32 with round-to-nearest-even, and, for bfloat16 storage, rounded
again from the float32 bits to bfloat16 with round-to-nearest-even.  The
float64 up-casts of the stored bits are returned beside them, so an fp64
consumer sees exactly what the device sees.

Workload shapes follow the Performer paper pages: sequences up to and
beyond 4096 tokens, head dimension d, and m random features drawn as
stacked d x d orthogonal blocks ("Masked Language Modeling for Proteins
via Linearly Scalable Long-Context Transformers", Methodology and
Experimental Design sections; the FAVOR+ blog page, section on the FAVOR+
core mechanism).  The datasets the pages train on (UniRef, Pfam,
ImageNet64) are not used: every tensor is synthetic with the stated
distribution.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

# One PCG64 stream per tensor so that changing one tensor's shape never
# shifts another tensor's values.
STREAM: Dict[str, int] = {
    "omega": 0,      # Gaussian d x d blocks for the orthogonal features
    "q": 1,
    "k": 2,
    "v": 3,
    "radii": 4,      # chi(d) row norms for the orthogonal features
    "ids": 5,        # protein-like token ids
    "mask": 6,       # masked-LM replacement draws
    "embed": 7,
    "wq": 8,
    "wk": 9,
    "wv": 10,
    "wo": 11,
    "rows": 12,      # sampled output rows for long-sequence checks
    "qnorm": 13,     # row radii for the norm-shell distribution (queries)
    "knorm": 14,     # row radii for the norm-shell distribution (keys)
    "dout": 15,      # upstream gradient of the output (backward pass)
}

DTYPES = ("f32", "bf16")


def rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), STREAM[stream]])


# ---------------------------------------------------------------- storage
def f32_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to float32 (round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest even.

    Finite inputs only (the generators never produce inf or NaN)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str):
    """(stored array, exact float64 view of what was stored)."""
    x32 = f32_round(x64)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(x32)
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------- random features
@dataclasses.dataclass
class OmegaDraws:
    """Raw draws from which an orthogonal random-feature matrix is built.

    gaussian: [n_blocks, d, d] i.i.d. N(0, 1); radii: [m] chi(d) draws.
    Building the matrix (orthogonalise each block's rows, rescale each
    row to its radius, stack, keep the first m rows) is a step of the
    method and is done separately by each consumer."""
    gaussian: np.ndarray
    radii: np.ndarray
    m: int
    d: int


def omega_draws(m: int, d: int, seed: int = 0) -> OmegaDraws:
    if m < 1 or d < 1:
        raise ValueError("m and d must be positive")
    n_blocks = -(-m // d)
    g = rng(seed, "omega").standard_normal((n_blocks, d, d))
    # chi(d) variates: square root of chi-square(d) draws.
    radii = np.sqrt(rng(seed, "radii").chisquare(d, size=m))
    return OmegaDraws(gaussian=g, radii=radii, m=m, d=d)


def iid_gaussian_omega(m: int, d: int, seed: int) -> np.ndarray:
    """Unstructured (i.i.d. N(0,1)) random features, the ablation baseline
    that orthogonal features are compared against."""
    return rng(seed, "omega").standard_normal((m, d))


# ---------------------------------------------------------- attention io
@dataclasses.dataclass
class AttentionInputs:
    B: int
    H: int
    L: int
    d: int
    dtype: str
    q: np.ndarray     # storage: float32 or uint16 (bf16 bits), [B,H,L,d]
    k: np.ndarray
    v: np.ndarray
    q64: np.ndarray   # exact float64 value of the stored bits
    k64: np.ndarray
    v64: np.ndarray


def _gaussian_rows(shape, d, seed, stream):
    return rng(seed, stream).standard_normal(shape) * d ** -0.25


def _norm_shell_rows(shape, seed, stream, radius_stream, lo=0.5, hi=2.0):
    g = rng(seed, stream).standard_normal(shape)
    r = rng(seed, radius_stream).uniform(lo, hi, size=shape[:-1])
    return g / np.linalg.norm(g, axis=-1, keepdims=True) * r[..., None]


def attention_inputs(B: int, H: int, L: int, d: int, dtype: str, seed: int = 0,
                     norm_shells: bool = False) -> AttentionInputs:
    """Q, K, V of shape [B, H, L, d].

    Default: i.i.d. N(0, 1) * d**-0.25.  With ``norm_shells`` the rows of
    Q and K are uniformly random directions with norms uniform in
    [0.5, 2] (V keeps the default distribution)."""
    shape = (B, H, L, d)
    if norm_shells:
        q = _norm_shell_rows(shape, seed, "q", "qnorm")
        k = _norm_shell_rows(shape, seed, "k", "knorm")
    else:
        q = _gaussian_rows(shape, d, seed, "q")
        k = _gaussian_rows(shape, d, seed, "k")
    v = _gaussian_rows(shape, d, seed, "v")
    qs, q64 = to_storage(q, dtype)
    ks, k64 = to_storage(k, dtype)
    vs, v64 = to_storage(v, dtype)
    return AttentionInputs(B, H, L, d, dtype, qs, ks, vs, q64, k64, v64)


def output_grads(B: int, H: int, L: int, d: int, dtype: str, seed: int = 0):
    """dL/d out of shape [B, H, L, d]: i.i.d. N(0, 1), stored like the
    inputs; returns (stored array, exact float64 view)."""
    g = rng(seed, "dout").standard_normal((B, H, L, d))
    return to_storage(g, dtype)


def sample_rows(L: int, n: int = 256, seed: int = 0) -> np.ndarray:
    """Sorted distinct output rows: {0, 1, 2, 3, L-1} plus uniform draws."""
    fixed = sorted({r for r in (0, 1, 2, 3, L - 1) if 0 <= r < L})
    pool = np.setdiff1d(np.arange(L), fixed)
    extra = max(0, min(n - len(fixed), pool.size))
    draw = rng(seed, "rows").choice(pool, size=extra, replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), draw.astype(np.int64)]))


# ------------------------------------------------ masked-LM block inputs
@dataclasses.dataclass
class BlockInputs:
    B: int
    L: int
    E: int
    H: int
    vocab: int
    mask_id: int
    ids: np.ndarray          # int32 [B, L]
    embed: np.ndarray        # bf16 bits [vocab, E]
    wq: np.ndarray           # bf16 bits [E, E]  (Y = X @ W)
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    embed64: np.ndarray
    wq64: np.ndarray
    wk64: np.ndarray
    wv64: np.ndarray
    wo64: np.ndarray


def block_inputs(B: int = 2, L: int = 4096, E: int = 512, H: int = 8, seed: int = 0,
                 alphabet: int = 25, mask_rate: float = 0.15, init_std: float = 0.02) -> BlockInputs:
    """Protein-like masked-LM block inputs: token ids uniform over a
    25-symbol alphabet with each position independently replaced by a
    mask id with probability 0.15; embedding and projection weights
    N(0, init_std**2), stored as bfloat16."""
    ids = rng(seed, "ids").integers(0, alphabet, size=(B, L))
    mask = rng(seed, "mask").random((B, L)) < mask_rate
    ids = np.where(mask, alphabet, ids).astype(np.int32)
    vocab = alphabet + 1
    emb, emb64 = to_storage(rng(seed, "embed").standard_normal((vocab, E)) * init_std, "bf16")
    ws = {}
    for name in ("wq", "wk", "wv", "wo"):
        ws[name] = to_storage(rng(seed, name).standard_normal((E, E)) * init_std, "bf16")
    return BlockInputs(B, L, E, H, vocab, alphabet, ids, emb,
                       ws["wq"][0], ws["wk"][0], ws["wv"][0], ws["wo"][0],
                       emb64, ws["wq"][1], ws["wk"][1], ws["wv"][1], ws["wo"][1])


# ------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    m: int
    dtype: str
    kind: str                # "trig" | "relu" | "positive"
    causal: bool
    norm_shells: bool = False
    sampled_rows: Optional[int] = None   # oracle checks only these rows

    @property
    def tokens_x_heads(self) -> int:
        return self.B * self.H * self.L


WORKLOADS: Dict[str, Workload] = {
    # Small fp32 case: Omega is 4 stacked 16 x 16 blocks.
    "c1": Workload("c1", 1, 1, 512, 16, 64, "f32", "trig", False),
    "c2_trig": Workload("c2_trig", 8, 8, 1024, 64, 256, "bf16", "trig", False),
    "c2_relu": Workload("c2_relu", 8, 8, 1024, 64, 256, "bf16", "relu", False),
    "c3_causal": Workload("c3_causal", 4, 8, 4096, 64, 256, "bf16", "trig", True),
    # Headline shape: the causal case's shape, run bidirectionally.
    "head": Workload("head", 4, 8, 4096, 64, 256, "bf16", "trig", False),
    "c4_bidir": Workload("c4_bidir", 1, 8, 32768, 64, 256, "bf16", "trig", False, True, 256),
    "c4_causal": Workload("c4_causal", 1, 8, 32768, 64, 256, "bf16", "trig", True, True, 256),
    # The positive (softmax-kernel) map on the headline shape.
    "pos_bidir": Workload("pos_bidir", 4, 8, 4096, 64, 256, "bf16", "positive", False),
    "pos_causal": Workload("pos_causal", 4, 8, 4096, 64, 256, "bf16", "positive", True),
}

BLOCK_WORKLOAD = dict(B=2, L=4096, E=512, H=8, d=64, m=256, kind="relu", dtype="bf16")


def workload_inputs(w: Workload, seed: int = 0):
    """(AttentionInputs, OmegaDraws) for a named workload."""
    return (attention_inputs(w.B, w.H, w.L, w.d, w.dtype, seed, w.norm_shells),
            omega_draws(w.m, w.d, seed))
