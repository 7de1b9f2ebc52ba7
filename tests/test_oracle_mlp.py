"""Pins of the oracle's two-layer inner model f(x) = W2 silu(W1 x)
("Edifice.Recurrent.TTT", Options, `:variant`: a hidden state that is a
two-layer MLP; "Error Correction in Trained TTT Layers", abstract: TTT-MLP
under the LayerNorm squared-error objective).

Each inner step's gradients are checked against torch autograd of the loss
(the straight-through mode through a detached LayerNorm residual) and against
central finite differences; the whole scan against an independent torch scan
that takes every step's gradient by autograd; the eta -> 0 limit against the
frozen-model closed form; the dual form with chunk 1 against the per-token
scan; and the first dual chunk against per-token gradients taken at W0."""
import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import make_mlp_case

torch = pytest.importorskip("torch")


def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


def _torch_loss(W1, W2, k, v, gamma, beta, ln, eps=oracle.EPS):
    """0.5 ||LN(W2 silu(W1 k)) - v||^2 written with torch ops; in the
    straight-through mode the LayerNorm enters as z + stopgrad(LN(z) - z)."""
    a = torch.nn.functional.silu(W1 @ k)
    z = W2 @ a
    if ln == "none":
        pred = z
    else:
        ln_z = torch.nn.functional.layer_norm(z, z.shape, weight=gamma, bias=beta, eps=eps)
        pred = ln_z if ln == "exact" else z + (ln_z - z).detach()
    return 0.5 * ((pred - v) ** 2).sum()


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("d", [1, 3, 8])
def test_inner_grads_match_autograd(ln, d):
    W1, W2 = _rand((d, d), 1, 0.7), _rand((d, d), 2, 0.5)
    k, v = _rand(d, 3), _rand(d, 4)
    gamma, beta = 1.0 + _rand(d, 5, 0.2), _rand(d, 6, 0.2)
    t = [torch.tensor(a, requires_grad=i < 2) for i, a in enumerate((W1, W2, k, v, gamma, beta))]
    _torch_loss(*t, ln).backward()
    g1, g2 = oracle.mlp_inner_grads(W1, W2, k, v, gamma, beta, ln)
    np.testing.assert_allclose(g1, t[0].grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2, t[1].grad.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("ln", ["exact", "none"])
def test_inner_grads_match_finite_differences(ln):
    d = 5
    W1, W2 = _rand((d, d), 11, 0.8), _rand((d, d), 12, 0.6)
    k, v = _rand(d, 13), _rand(d, 14)
    gamma, beta = 1.0 + _rand(d, 15, 0.2), _rand(d, 16, 0.2)

    def loss(A, B):
        z = B @ oracle.silu(A @ k)
        pred = z if ln == "none" else oracle.layer_norm(z, gamma, beta)[0]
        return 0.5 * float(((pred - v) ** 2).sum())

    g1, g2 = oracle.mlp_inner_grads(W1, W2, k, v, gamma, beta, ln)
    h = 1e-6
    for W, g, which in ((W1, g1, 0), (W2, g2, 1)):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            p, m = W.copy(), W.copy()
            p[idx] += h
            m[idx] -= h
            args_p = (p, W2) if which == 0 else (W1, p)
            args_m = (m, W2) if which == 0 else (W1, m)
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def _torch_scan(c, W1, ln, dual, chunk):
    """An independent scan: torch float64, each step's gradients by autograd."""
    T64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    q, k, v, eta, gate = map(T64, (c.q, c.k, c.v, c.eta_logit, c.gate_logit))
    B, H, T, d = c.q.shape
    out = torch.zeros(B, H, T, d, dtype=torch.float64)
    W1f = T64(W1).clone()
    W2f = T64(c.W0).clone()
    for b in range(B):
        for h in range(H):
            gam, bet = T64(c.gamma[h]), T64(c.beta[h])
            A, Bm = W1f[b, h].clone(), W2f[b, h].clone()
            for t in range(T):
                if not dual or t % chunk == 0:
                    PA = A.clone().requires_grad_(True)
                    PB = Bm.clone().requires_grad_(True)
                if dual:
                    PA.grad = None
                    PB.grad = None
                loss = _torch_loss(PA, PB, k[b, h, t], v[b, h, t], gam, bet, ln)
                gA, gB = torch.autograd.grad(loss, (PA, PB))
                lr = torch.sigmoid(eta[b, h, t]) / d
                A = A - lr * gA
                Bm = Bm - lr * gB
                if not dual:
                    PA = A.clone().requires_grad_(True)
                    PB = Bm.clone().requires_grad_(True)
                y = Bm @ torch.nn.functional.silu(A @ q[b, h, t])
                out[b, h, t] = y * torch.sigmoid(gate[b, h, t])
            W1f[b, h], W2f[b, h] = A, Bm
    return out.numpy(), W1f.numpy(), W2f.numpy()


@pytest.mark.parametrize("ln,dual,chunk", [("st", False, 16), ("exact", False, 16),
                                           ("none", False, 16), ("st", True, 4),
                                           ("exact", True, 3), ("none", True, 5)])
def test_scan_matches_independent_torch_scan(ln, dual, chunk):
    c, W1 = make_mlp_case(2, 2, 11, 6, seed=31, ln=ln, random_affine=True)
    o, A, Bm = oracle.ttt_mlp_forward(c.q, c.k, c.v, c.eta_logit, c.gate_logit, W1, c.W0,
                                      c.gamma, c.beta, ln=ln, dual=dual, chunk=chunk)
    ro, rA, rB = _torch_scan(c, W1, ln, dual, chunk)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(A, rA, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(Bm, rB, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("dual", [False, True])
def test_frozen_model_when_eta_is_minus_infinity(dual):
    """sigmoid(-inf) = 0: no update, so o_t = (W2_0 silu(W1_0 q_t)) sigmoid(g_t)."""
    c, W1 = make_mlp_case(1, 3, 7, 5, seed=32)
    eta = np.full_like(c.eta_logit, -np.inf)
    o, A, Bm = oracle.ttt_mlp_forward(c.q, c.k, c.v, eta, c.gate_logit, W1, c.W0, c.gamma,
                                      c.beta, dual=dual, chunk=4)
    np.testing.assert_array_equal(A, W1.astype(np.float64))
    np.testing.assert_array_equal(Bm, c.W0.astype(np.float64))
    q = torch.tensor(c.q, dtype=torch.float64)
    hq = torch.einsum("bhij,bhtj->bhti", torch.tensor(W1, dtype=torch.float64), q)
    y = torch.einsum("bhij,bhtj->bhti", torch.tensor(c.W0, dtype=torch.float64),
                     torch.nn.functional.silu(hq))
    ref = (y * torch.sigmoid(torch.tensor(c.gate_logit, dtype=torch.float64))).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
def test_dual_with_chunk_one_is_per_token(ln):
    c, W1 = make_mlp_case(1, 2, 9, 4, seed=33, random_affine=True)
    args = (c.q, c.k, c.v, c.eta_logit, c.gate_logit, W1, c.W0, c.gamma, c.beta)
    r1 = oracle.ttt_mlp_forward(*args, ln=ln)
    r2 = oracle.ttt_mlp_forward(*args, ln=ln, dual=True, chunk=1)
    for a, b in zip(r1, r2):
        np.testing.assert_array_equal(a, b)


def test_first_dual_chunk_sums_gradients_taken_at_the_initial_weights():
    """Within the first chunk every gradient is taken at (W1_0, W2_0), so the
    weights after the chunk are W_0 minus the eta-weighted sum of T one-token
    gradients, each an independent per-token scan of length 1 started at W_0."""
    c, W1 = make_mlp_case(1, 1, 6, 5, seed=34)
    _, A, Bm = oracle.ttt_mlp_forward(c.q, c.k, c.v, c.eta_logit, c.gate_logit, W1, c.W0,
                                      c.gamma, c.beta, dual=True, chunk=6)
    sA, sB = W1.astype(np.float64).copy(), c.W0.astype(np.float64).copy()
    for t in range(6):
        sl = lambda a: a[:, :, t:t + 1]
        _, A1, B1 = oracle.ttt_mlp_forward(sl(c.q), sl(c.k), sl(c.v), c.eta_logit[:, :, t:t + 1],
                                           sl(c.gate_logit), W1, c.W0, c.gamma, c.beta)
        sA += A1 - W1
        sB += B1 - c.W0
    np.testing.assert_allclose(A, sA, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(Bm, sB, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("mistake", ["no_silu_grad", "linear_activation", "sign_of_delta"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    """A mistake planted in the oracle (a dropped silu' factor, the activation
    left out of dL/dW2, a flipped inner-gradient sign) fails the autograd pin."""
    mod = oracle.ttt_oracle
    if mistake == "no_silu_grad":
        monkeypatch.setattr(mod, "silu_grad", lambda x: np.ones_like(x))
    elif mistake == "linear_activation":
        monkeypatch.setattr(mod, "silu", lambda x: x)
    else:
        real = mod.inner_grad_vector
        monkeypatch.setattr(mod, "inner_grad_vector", lambda *a, **k: -real(*a, **k))
    d = 6
    W1, W2 = _rand((d, d), 41, 0.7), _rand((d, d), 42, 0.5)
    k, v = _rand(d, 43), _rand(d, 44)
    gamma, beta = 1.0 + _rand(d, 45, 0.2), _rand(d, 46, 0.2)
    t = [torch.tensor(a, requires_grad=i < 2) for i, a in enumerate((W1, W2, k, v, gamma, beta))]
    _torch_loss(*t, "exact").backward()
    g1, g2 = mod.mlp_inner_grads(W1, W2, k, v, gamma, beta, "exact")
    err = max(np.max(np.abs(g1 - t[0].grad.numpy())) / np.max(np.abs(t[0].grad.numpy())),
              np.max(np.abs(g2 - t[1].grad.numpy())) / np.max(np.abs(t[1].grad.numpy())))
    assert err > 1e-3
