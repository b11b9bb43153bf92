"""Plain float64 CPU oracle for FAVOR attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the GPU library is checked against.  Only the test suite,
the package smoke check and the CPU-baseline leg of the benchmark may
import it; the library's product path never does, and this module
imports nothing from the library (its inputs come from the seeded
generators, which hold no part of the method's arithmetic).

Sources (web pages about the Performer / FAVOR papers; cited by title and
section):

* [blog]  "用随机特征“骗”过 softmax，Transformer 注意力也能跑成线性？"
          (page on arXiv 2009.14794), section 核心机制：FAVOR+ .
* [en]    "Masked Language Modeling for Proteins via Linearly Scalable
          Long-Context Transformers", English summary page: sections
          Methodology, Technical Contribution, Limitations,
          AI Executive Summary.
* [zh]    the same paper's Chinese summary page: sections 方法论,
          核心创新, 方法详解, 实验设计.

What is computed (all float64, no blocking or fusion beyond what the
definitions state):

1. Orthogonal random features (ORF) [blog §核心机制：FAVOR+; zh §方法详解]:
   Omega's rows are a random sub-sample of an orthogonal matrix.  Each
   d x d block is a Gaussian matrix whose rows are orthogonalised by
   Gram-Schmidt in order and then rescaled to independent chi(d) norms,
   so that every row is marginally N(0, I_d); blocks are stacked and the
   first m rows kept.
2. Feature maps [blog §核心机制：FAVOR+; en §AI Executive Summary;
   zh §核心创新 item 2]:
     x~ = d**-0.25 * x,  P = x~ Omega^T  (L x m)
     trig: phi(x) = exp(|x~|^2 / 2) * m**-0.5 * [sin P, cos P]   (F = 2m)
     relu: phi(x) = m**-0.5 * max(P, 0)                          (F = m)
     positive: phi(x) = m**-0.5 * exp(P - |x~|^2 / 2)            (F = m)
   so that E[phi(q).phi(k)] = exp(q.k / sqrt(d)) for the trig and the
   positive maps.  The positive (non-negative) map is the FAVOR+ variant
   the blog section names but prints garbled; its form here follows from
   the Gaussian moment-generating function E_w[exp(w.a)] = exp(|a|^2 / 2)
   for w ~ N(0, I): E[exp(w.q~ - |q~|^2/2) exp(w.k~ - |k~|^2/2)] =
   exp(|q~ + k~|^2 / 2 - |q~|^2 / 2 - |k~|^2 / 2) = exp(q~.k~).
3. Bidirectional [blog §核心机制：FAVOR+]: S = phi(K)^T V, z = phi(K)^T 1,
   out_i = phi(q_i)^T S / phi(q_i)^T z.  No L x L matrix.
4. Causal [blog §核心机制：FAVOR+, causal variant]: the same with the
   inclusive prefix sums S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j).
5. Quadratic form (used to check 3 and 4): A_ij = phi(q_i).phi(k_j),
   zero for j > i when causal; out = (A V) / (A 1)  -- the D^-1 A V form
   of the same section with exp(q.k/sqrt(d)) replaced by phi(q).phi(k).
6. Textbook softmax attention D^-1 exp(Q K^T / sqrt(d)) V
   [blog §核心机制：FAVOR+], the large-m limit of 3 and 4.
7. Gradients of 3 and 4 (the pages claim training-time speedups [en
   §Methodology] but print no backward pass; this is the chain rule of
   the same computation).  For a loss with dL/d out_i = g_i:
     a_i = g_i / den_i,  b_i = -(g_i . out_i) / den_i     (dL/dnum, dL/dden)
     dphi(q_i) = S_i a_i + z_i b_i
     R_j = sum_{i >= j} phi(q_i) a_i^T,  r_j = sum_{i >= j} phi(q_i) b_i
           (all i for bidirectional: R = dL/dS, r = dL/dz)
     dv_j = R_j^T phi(k_j),  dphi(k_j) = R_j v_j + r_j
   and through each map (mu = m**-0.5, x~ = d**-0.25 x, upstream w):
     trig:     dP = c mu (w_sin cos P - w_cos sin P),  c = exp(|x~|^2/2);
               dx~ = Omega^T dP + (w . phi) x~
     relu:     dP = mu w [P > 0];  dx~ = Omega^T dP
     positive: dP = w * phi;  dx~ = Omega^T dP - (w . phi) x~
     dx = d**-0.25 dx~.

Readings where the pages are silent (each is listed with its reason in
the design notes): d**-0.25 is applied inside phi to the tensors passed
in; m counts the rows of Omega; the causal prefix is inclusive; the
denominator has no epsilon; relu is the generalized-attention map with
f = ReLU and no extra scaling.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional, Sequence

import numpy as np

KINDS = ("trig", "relu", "positive")


# --------------------------------------------------------------- step 1
def gram_schmidt_rows(G: np.ndarray) -> np.ndarray:
    """Orthonormalise the rows of G in order (modified Gram-Schmidt)."""
    G = np.array(G, dtype=np.float64, copy=True)
    n = G.shape[0]
    for r in range(n):
        for s in range(r):
            G[r] -= (G[r] @ G[s]) * G[s]
        G[r] /= np.linalg.norm(G[r])
    return G


def orthogonal_random_features(gaussian: np.ndarray, radii: np.ndarray, m: int) -> np.ndarray:
    """Omega [m, d]: stacked orthogonalised Gaussian blocks, rows rescaled
    to the given chi(d) radii [blog §核心机制：FAVOR+; zh §方法详解]."""
    gaussian = np.asarray(gaussian, dtype=np.float64)
    n_blocks, d, d2 = gaussian.shape
    if d != d2 or n_blocks * d < m:
        raise ValueError("need n_blocks * d >= m square blocks")
    rows = np.concatenate([gram_schmidt_rows(gaussian[b]) for b in range(n_blocks)], axis=0)[:m]
    return rows * np.asarray(radii, dtype=np.float64)[:m, None]


# --------------------------------------------------------------- step 2
def feature_width(m: int, kind: str) -> int:
    return 2 * m if kind == "trig" else m


def feature_map(X: np.ndarray, Omega: np.ndarray, kind: str) -> np.ndarray:
    """phi(X) for X [..., L, d] -> [..., L, F]."""
    X = np.asarray(X, dtype=np.float64)
    Omega = np.asarray(Omega, dtype=np.float64)
    d = X.shape[-1]
    m = Omega.shape[0]
    Xt = X * d ** -0.25
    P = Xt @ Omega.T
    if kind == "trig":
        half_sq_norm = 0.5 * np.sum(Xt * Xt, axis=-1, keepdims=True)
        return np.exp(half_sq_norm) * m ** -0.5 * np.concatenate([np.sin(P), np.cos(P)], axis=-1)
    if kind == "relu":
        return m ** -0.5 * np.maximum(P, 0.0)
    if kind == "positive":
        half_sq_norm = 0.5 * np.sum(Xt * Xt, axis=-1, keepdims=True)
        return m ** -0.5 * np.exp(P - half_sq_norm)
    raise ValueError(f"unknown feature kind {kind!r}")


# --------------------------------------------------------- steps 3 and 4
def _bidirectional_head(q, k, v, Omega, kind):
    phq = feature_map(q, Omega, kind)
    phk = feature_map(k, Omega, kind)
    S = phk.T @ v                 # [F, d]
    z = phk.sum(axis=0)           # [F]
    return (phq @ S) / (phq @ z)[:, None]


def _causal_head(q, k, v, Omega, kind, block=256):
    phq = feature_map(q, Omega, kind)
    phk = feature_map(k, Omega, kind)
    L, F = phk.shape
    d = v.shape[1]
    S = np.zeros((F, d))
    z = np.zeros(F)
    out = np.empty((L, d))
    for t0 in range(0, L, block):
        t1 = min(L, t0 + block)
        # inclusive prefix: S_i = S_carry + sum_{t0 <= j <= i} phi(k_j) v_j^T
        Si = S + np.cumsum(phk[t0:t1, :, None] * v[t0:t1, None, :], axis=0)
        zi = z + np.cumsum(phk[t0:t1], axis=0)
        num = np.einsum("tf,tfd->td", phq[t0:t1], Si)
        den = np.einsum("tf,tf->t", phq[t0:t1], zi)
        out[t0:t1] = num / den[:, None]
        S = Si[-1]
        z = zi[-1]
    return out


def _map_heads(fn, Q, K, V, workers):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Q.shape[:-2]
    L, d = Q.shape[-2:]
    q2 = Q.reshape(-1, L, d)
    k2 = K.reshape(-1, K.shape[-2], d)
    v2 = V.reshape(-1, V.shape[-2], V.shape[-1])
    n = q2.shape[0]
    out = np.empty((n, L, v2.shape[-1]))
    if workers and workers > 1 and n > 1:
        with ThreadPoolExecutor(max_workers=min(workers, n)) as ex:
            for i, o in enumerate(ex.map(lambda i: fn(q2[i], k2[i], v2[i]), range(n))):
                out[i] = o
    else:
        for i in range(n):
            out[i] = fn(q2[i], k2[i], v2[i])
    return out.reshape(*lead, L, v2.shape[-1])


def favor_attention(Q, K, V, Omega, kind: str = "trig", causal: bool = False,
                    workers: Optional[int] = None) -> np.ndarray:
    """Linear-order FAVOR attention on [..., L, d] inputs (float64)."""
    if kind not in KINDS:
        raise ValueError(f"unknown feature kind {kind!r}")
    if causal:
        return _map_heads(lambda q, k, v: _causal_head(q, k, v, Omega, kind), Q, K, V, workers)
    return _map_heads(lambda q, k, v: _bidirectional_head(q, k, v, Omega, kind), Q, K, V, workers)


# --------------------------------------------------------------- step 5
def favor_quadratic(Q, K, V, Omega, kind: str = "trig", causal: bool = False) -> np.ndarray:
    """D^-1 A V with A_ij = phi(q_i).phi(k_j) formed explicitly (L x L)."""
    phq = feature_map(Q, Omega, kind)
    phk = feature_map(K, Omega, kind)
    A = phq @ np.swapaxes(phk, -1, -2)
    if causal:
        L = A.shape[-1]
        A = A * np.tril(np.ones((L, L)))
    return (A @ np.asarray(V, dtype=np.float64)) / A.sum(axis=-1, keepdims=True)


def favor_rows(Q, K, V, Omega, kind: str, causal: bool, rows: Sequence[int]) -> np.ndarray:
    """Output rows ``rows`` of every head, [..., len(rows), d].

    Bidirectional: the full S, z, read out only at the given rows.
    Causal: the inclusive prefix state, advanced key by key range in
    increasing row order and read out at each requested row."""
    rows = np.asarray(rows, dtype=np.int64)
    order = np.argsort(rows, kind="stable")
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Q.shape[:-2]
    L, d = Q.shape[-2:]
    dv = V.shape[-1]
    q2, k2, v2 = Q.reshape(-1, L, d), K.reshape(-1, L, d), V.reshape(-1, L, dv)
    out = np.empty((q2.shape[0], rows.size, dv))
    for h in range(q2.shape[0]):
        phq = feature_map(q2[h][rows], Omega, kind)
        phk = feature_map(k2[h], Omega, kind)
        if not causal:
            S = phk.T @ v2[h]
            z = phk.sum(axis=0)
            out[h] = (phq @ S) / (phq @ z)[:, None]
            continue
        S = np.zeros((phk.shape[1], dv))
        z = np.zeros(phk.shape[1])
        prev = 0
        for idx in order:
            r = int(rows[idx])
            if r + 1 > prev:
                S = S + phk[prev:r + 1].T @ v2[h][prev:r + 1]
                z = z + phk[prev:r + 1].sum(axis=0)
                prev = r + 1
            out[h, idx] = (phq[idx] @ S) / (phq[idx] @ z)
    return out.reshape(*lead, rows.size, dv)


def favor_quadratic_rows(Q, K, V, Omega, kind: str, causal: bool, rows: Sequence[int]) -> np.ndarray:
    """Rows of the explicit D^-1 A V form, one A row at a time."""
    rows = np.asarray(rows, dtype=np.int64)
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Q.shape[:-2]
    L, d = Q.shape[-2:]
    dv = V.shape[-1]
    q2, k2, v2 = Q.reshape(-1, L, d), K.reshape(-1, L, d), V.reshape(-1, L, dv)
    out = np.empty((q2.shape[0], rows.size, dv))
    for h in range(q2.shape[0]):
        phq = feature_map(q2[h][rows], Omega, kind)
        phk = feature_map(k2[h], Omega, kind)
        A = phq @ phk.T                     # [len(rows), L]
        if causal:
            A = A * (np.arange(L)[None, :] <= rows[:, None])
        out[h] = (A @ v2[h]) / A.sum(axis=1, keepdims=True)
    return out.reshape(*lead, rows.size, dv)


# --------------------------------------------------------------- step 6
def softmax_attention(Q, K, V, causal: bool = False) -> np.ndarray:
    """D^-1 A V with A = exp(Q K^T / sqrt(d)) [blog §核心机制：FAVOR+]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    d = Q.shape[-1]
    A = np.exp(Q @ np.swapaxes(K, -1, -2) / np.sqrt(d))
    if causal:
        L = A.shape[-1]
        A = A * np.tril(np.ones((L, L)))
    return (A @ np.asarray(V, dtype=np.float64)) / A.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------- step 7
def feature_map_vjp(X: np.ndarray, Omega: np.ndarray, kind: str, dphi: np.ndarray) -> np.ndarray:
    """dL/dX given dL/dphi(X) = dphi (X [..., L, d], dphi [..., L, F]):
    the chain rule through x~ = d^-1/4 x, P = x~ Omega^T and the map.
    ReLU takes derivative 0 at P = 0."""
    X = np.asarray(X, dtype=np.float64)
    Omega = np.asarray(Omega, dtype=np.float64)
    w = np.asarray(dphi, dtype=np.float64)
    d = X.shape[-1]
    m = Omega.shape[0]
    mu = m ** -0.5
    Xt = X * d ** -0.25
    P = Xt @ Omega.T
    if kind == "trig":
        c = np.exp(0.5 * np.sum(Xt * Xt, axis=-1, keepdims=True))
        ws, wc = w[..., :m], w[..., m:]
        dP = c * mu * (ws * np.cos(P) - wc * np.sin(P))
        phi = c * mu * np.concatenate([np.sin(P), np.cos(P)], axis=-1)
        dXt = dP @ Omega + np.sum(w * phi, axis=-1, keepdims=True) * Xt
    elif kind == "relu":
        dP = mu * w * (P > 0.0)
        dXt = dP @ Omega
    elif kind == "positive":
        phi = mu * np.exp(P - 0.5 * np.sum(Xt * Xt, axis=-1, keepdims=True))
        dP = w * phi
        dXt = dP @ Omega - np.sum(dP, axis=-1, keepdims=True) * Xt
    else:
        raise ValueError(f"unknown feature kind {kind!r}")
    return dXt * d ** -0.25


def _bidirectional_head_grad(q, k, v, g, Omega, kind):
    phq = feature_map(q, Omega, kind)
    phk = feature_map(k, Omega, kind)
    S = phk.T @ v
    z = phk.sum(axis=0)
    den = phq @ z
    out = (phq @ S) / den[:, None]
    a = g / den[:, None]
    b = -np.sum(g * out, axis=1) / den
    dphq = a @ S.T + b[:, None] * z[None, :]
    R = phq.T @ a                 # dL/dS  [F, d]
    r = phq.T @ b                 # dL/dz  [F]
    dv = phk @ R
    dphk = v @ R.T + r[None, :]
    return feature_map_vjp(q, Omega, kind, dphq), feature_map_vjp(k, Omega, kind, dphk), dv


def _causal_head_grad(q, k, v, g, Omega, kind, block=64):
    phq = feature_map(q, Omega, kind)
    phk = feature_map(k, Omega, kind)
    L, F = phk.shape
    d = v.shape[1]
    a = np.empty((L, d))
    b = np.empty(L)
    dphq = np.empty((L, F))
    # forward prefix states S_i, z_i (inclusive), block by block
    S = np.zeros((F, d))
    z = np.zeros(F)
    for t0 in range(0, L, block):
        t1 = min(L, t0 + block)
        Si = S + np.cumsum(phk[t0:t1, :, None] * v[t0:t1, None, :], axis=0)
        zi = z + np.cumsum(phk[t0:t1], axis=0)
        den = np.einsum("tf,tf->t", phq[t0:t1], zi)
        out = np.einsum("tf,tfd->td", phq[t0:t1], Si) / den[:, None]
        a[t0:t1] = g[t0:t1] / den[:, None]
        b[t0:t1] = -np.sum(g[t0:t1] * out, axis=1) / den
        dphq[t0:t1] = np.einsum("tfd,td->tf", Si, a[t0:t1]) + zi * b[t0:t1, None]
        S, z = Si[-1], zi[-1]
    # suffix sums R_j = sum_{i >= j} phi(q_i) a_i^T, r_j likewise, from the end
    dv = np.empty((L, d))
    dphk = np.empty((L, F))
    R = np.zeros((F, d))
    r = np.zeros(F)
    for t1 in range(L, 0, -block):
        t0 = max(0, t1 - block)
        Rj = R + np.cumsum((phq[t0:t1, :, None] * a[t0:t1, None, :])[::-1], axis=0)[::-1]
        rj = r + np.cumsum((phq[t0:t1] * b[t0:t1, None])[::-1], axis=0)[::-1]
        dv[t0:t1] = np.einsum("tfd,tf->td", Rj, phk[t0:t1])
        dphk[t0:t1] = np.einsum("tfd,td->tf", Rj, v[t0:t1]) + rj
        R, r = Rj[0], rj[0]
    return feature_map_vjp(q, Omega, kind, dphq), feature_map_vjp(k, Omega, kind, dphk), dv


def favor_attention_grad(Q, K, V, Omega, dOut, kind: str = "trig", causal: bool = False,
                         workers: Optional[int] = None):
    """(dQ, dK, dV) of L = sum(dOut * favor_attention(Q, K, V)) on [..., L, d]
    inputs (float64); Omega is fixed."""
    if kind not in KINDS:
        raise ValueError(f"unknown feature kind {kind!r}")
    Q, K, V, G = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dOut))
    lead = Q.shape[:-2]
    L, d = Q.shape[-2:]
    q2, k2, v2, g2 = (x.reshape(-1, L, d) for x in (Q, K, V, G))
    fn = _causal_head_grad if causal else _bidirectional_head_grad
    n = q2.shape[0]
    res = [None] * n
    if workers and workers > 1 and n > 1:
        with ThreadPoolExecutor(max_workers=min(workers, n)) as ex:
            res = list(ex.map(lambda i: fn(q2[i], k2[i], v2[i], g2[i], Omega, kind), range(n)))
    else:
        res = [fn(q2[i], k2[i], v2[i], g2[i], Omega, kind) for i in range(n)]
    return tuple(np.stack([r_[j] for r_ in res]).reshape(*lead, L, d) for j in range(3))


# ------------------------------------------------ masked-LM attention block
def performer_block(ids, embed, wq, wk, wv, wo, Omega, heads: int, kind: str = "relu",
                    workers: Optional[int] = None) -> np.ndarray:
    """One Performer attention block of a protein masked-LM
    [en §Methodology; zh §实验设计]: X = E[ids]; Q, K, V = X W_{q,k,v}
    split into heads (head h takes columns [h*dh, (h+1)*dh)); bidirectional
    FAVOR per head; Y = concat(heads) W_o.  No positional encoding and no
    normalisation layer (none is specified for this block)."""
    X = np.asarray(embed, dtype=np.float64)[np.asarray(ids)]
    B, L, E = X.shape
    dh = E // heads

    def split(Y):
        return Y.reshape(B, L, heads, dh).transpose(0, 2, 1, 3)

    Q = split(X @ np.asarray(wq, dtype=np.float64))
    K = split(X @ np.asarray(wk, dtype=np.float64))
    V = split(X @ np.asarray(wv, dtype=np.float64))
    O = favor_attention(Q, K, V, Omega, kind, causal=False, workers=workers)
    O = O.transpose(0, 2, 1, 3).reshape(B, L, E)
    return O @ np.asarray(wo, dtype=np.float64)


def default_workers() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
