"""Pins for the oracle's gradients (favor_attention_grad, feature_map_vjp).

The backward pass is the chain rule of the forward computation; it is
pinned against things other than its own formulas:
  * central finite differences of the forward oracle (float64);
  * torch autograd of an independently written quadratic form
    D^-1 A V with A = phi(Q) phi(K)^T (masked for causal);
  * exact identities: the attention weights of a row sum to one, so
    sum_j dV_j = sum_i dOut_i; the ReLU map is positively homogeneous in
    each query row, so q_i . dq_i = 0;
  * planted mistakes (a dropped term, a wrong sign, a prefix instead of a
    suffix) that each of these must reject."""
import numpy as np
import pytest
import torch

from oracle import favor_oracle as O


CASES = [(kind, causal) for kind in O.KINDS for causal in (False, True)]


def _problem(seed, B=1, H=2, L=9, d=4, m=6):
    """Random inputs whose every denominator phi(q_i).z_i is nonzero for all
    maps and both directions (ReLU rows with no overlap are 0/0, and their
    gradient is undefined), redrawn from the next seed until they are."""
    for s in range(seed, seed + 100):
        rng = np.random.default_rng(s)
        q, k, v, g = (rng.standard_normal((B, H, L, d)) for _ in range(4))
        W = rng.standard_normal((m, d))
        with np.errstate(invalid="ignore", divide="ignore"):
            ok = all(np.isfinite(O.favor_attention(q, k, v, W, kind, causal)).all()
                     and np.min(np.abs(O.feature_map(q, W, kind)
                                       @ np.swapaxes(O.feature_map(k, W, kind), -1, -2)).max(-1)) > 1e-3
                     for kind in O.KINDS for causal in (False, True))
        if ok:
            return q, k, v, g, W
    raise RuntimeError("no admissible draw")


def _fd_check(q, k, v, g, W, kind, causal, grads, n_dirs=3, h=1e-6, seed=1):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, x, dx in zip("qkv", (q, k, v), grads):
        for _ in range(n_dirs):
            e = rng.standard_normal(x.shape)

            def loss(xx):
                a = {"q": q, "k": k, "v": v}
                a[name] = xx
                return np.sum(g * O.favor_attention(a["q"], a["k"], a["v"], W, kind, causal))

            fd = (loss(x + h * e) - loss(x - h * e)) / (2 * h)
            an = float(np.sum(dx * e))
            worst = max(worst, abs(fd - an) / max(abs(an), 1e-8))
    return worst


@pytest.mark.parametrize("kind,causal", CASES)
def test_grad_matches_finite_differences(kind, causal):
    q, k, v, g, W = _problem(3)
    grads = O.favor_attention_grad(q, k, v, W, g, kind, causal)
    assert _fd_check(q, k, v, g, W, kind, causal, grads) < 1e-6


def _torch_phi(x, W, kind):
    d = x.shape[-1]
    m = W.shape[0]
    xt = x * d ** -0.25
    P = xt @ W.T
    if kind == "trig":
        c = torch.exp(0.5 * (xt * xt).sum(-1, keepdim=True))
        return c * m ** -0.5 * torch.cat([torch.sin(P), torch.cos(P)], -1)
    if kind == "relu":
        return m ** -0.5 * torch.relu(P)
    return m ** -0.5 * torch.exp(P - 0.5 * (xt * xt).sum(-1, keepdim=True))


@pytest.mark.parametrize("kind,causal", CASES)
def test_grad_matches_autograd_of_quadratic_form(kind, causal):
    q, k, v, g, W = _problem(5, L=11)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tW = torch.tensor(W, dtype=torch.float64)
    A = _torch_phi(tq, tW, kind) @ _torch_phi(tk, tW, kind).transpose(-1, -2)
    if causal:
        A = A * torch.tril(torch.ones(A.shape[-2:], dtype=torch.float64))
    out = (A @ tv) / A.sum(-1, keepdim=True)
    (out * torch.tensor(g)).sum().backward()
    ours = O.favor_attention_grad(q, k, v, W, g, kind, causal)
    for mine, ref in zip(ours, (tq.grad, tk.grad, tv.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-9 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("kind,causal", CASES)
def test_value_gradient_sums_to_output_gradient(kind, causal):
    q, k, v, g, W = _problem(7, L=13)
    _, _, dv = O.favor_attention_grad(q, k, v, W, g, kind, causal)
    np.testing.assert_allclose(dv.sum(axis=-2), g.sum(axis=-2), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_relu_query_gradient_is_orthogonal_to_query(causal):
    q, k, v, g, W = _problem(8, L=10)
    dq, _, _ = O.favor_attention_grad(q, k, v, W, g, "relu", causal)
    dots = np.sum(q * dq, axis=-1)
    assert np.max(np.abs(dots)) < 1e-10 * max(1.0, np.max(np.abs(dq)))


def test_grad_of_single_token_is_value_passthrough():
    # one token: out = v, so dV = dOut and dQ = dK = 0
    q, k, v, g, W = _problem(9, L=1)
    for kind in O.KINDS:
        for causal in (False, True):
            dq, dk, dv = O.favor_attention_grad(q, k, v, W, g, kind, causal)
            np.testing.assert_allclose(dv, g, rtol=1e-12)
            assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


# ------------------------------------------------------------ mutations
def _mutant_vjp(mode):
    base = O.feature_map_vjp

    def vjp(X, Omega, kind, dphi):
        X = np.asarray(X, dtype=np.float64)
        w = np.asarray(dphi, dtype=np.float64)
        d = X.shape[-1]
        m = Omega.shape[0]
        Xt = X * d ** -0.25
        P = Xt @ Omega.T
        if kind != "trig":
            return base(X, Omega, kind, dphi)
        c = np.exp(0.5 * np.sum(Xt * Xt, axis=-1, keepdims=True))
        ws, wc = w[..., :m], w[..., m:]
        sign = -1.0 if mode == "cos sign" else 1.0
        dP = c * m ** -0.5 * (ws * np.cos(P) - sign * wc * np.sin(P))
        phi = c * m ** -0.5 * np.concatenate([np.sin(P), np.cos(P)], axis=-1)
        dXt = dP @ Omega
        if mode != "no norm term":
            dXt = dXt + np.sum(w * phi, axis=-1, keepdims=True) * Xt
        return dXt * d ** -0.25
    return vjp


def _mutant_bidir_no_den_term(q, k, v, g, Omega, kind):
    phq, phk = O.feature_map(q, Omega, kind), O.feature_map(k, Omega, kind)
    S, z = phk.T @ v, phk.sum(axis=0)
    den = phq @ z
    a = g / den[:, None]
    dphq = a @ S.T                      # dL/dden dropped
    R = phq.T @ a
    return (O.feature_map_vjp(q, Omega, kind, dphq), O.feature_map_vjp(k, Omega, kind, v @ R.T),
            phk @ R)


_CAUSAL_GRAD = O._causal_head_grad


def _mutant_causal_prefix_for_keys(q, k, v, g, Omega, kind):
    # uses the bidirectional key side (all queries) instead of the suffix
    dq, _, _ = _CAUSAL_GRAD(q, k, v, g, Omega, kind)
    _, dk, dv = O._bidirectional_head_grad(q, k, v, g, Omega, kind)
    return dq, dk, dv


@pytest.mark.parametrize("mutant", ["no norm term", "cos sign", "no den term", "causal keys see all"])
def test_pins_reject_planted_mistakes(monkeypatch, mutant):
    causal = mutant == "causal keys see all"
    if mutant in ("no norm term", "cos sign"):
        monkeypatch.setattr(O, "feature_map_vjp", _mutant_vjp(mutant))
    elif mutant == "no den term":
        monkeypatch.setattr(O, "_bidirectional_head_grad", _mutant_bidir_no_den_term)
    else:
        monkeypatch.setattr(O, "_causal_head_grad", _mutant_causal_prefix_for_keys)
    q, k, v, g, W = _problem(3)
    grads = O.favor_attention_grad(q, k, v, W, g, "trig", causal)
    assert _fd_check(q, k, v, g, W, "trig", causal, grads) > 1e-3
