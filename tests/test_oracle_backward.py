"""Pins of the oracle's backward pass (CPU, float64).

``oracle.ttt_linear_backward`` is checked against three things that do not
share its derivation:

* central finite differences of the forward (every input element, tiny sizes);
* torch autograd through an independent float64 torch forward written here
  (``torch.nn.functional.layer_norm``; the exact inner gradient itself taken by
  autograd with ``create_graph=True``, so the backward differentiates through
  a gradient);
* the closed form at eta -> 0 (eta_logit = -inf), where W stays W0.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

MODES = [("st", False, 1), ("exact", False, 1), ("none", False, 1),
         ("st", True, 2), ("exact", True, 3), ("none", True, 2), ("st", True, 8)]


def _case(B, H, T, d, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *s: rng.standard_normal(s)
    return dict(q=mk(B, H, T, d), k=mk(B, H, T, d), v=mk(B, H, T, d), eta_logit=mk(B, H, T),
                gate_logit=mk(B, H, T, d), W0=0.3 * mk(B, H, d, d), gamma=1 + 0.3 * mk(H, d),
                beta=0.3 * mk(H, d)), mk(B, H, T, d), mk(B, H, d, d)


GRADS = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("gate_logit", "dgate_logit"),
         ("eta_logit", "deta_logit"), ("W0", "dW0"), ("gamma", "dgamma"), ("beta", "dbeta")]


@pytest.mark.parametrize("ln,dual,chunk", MODES)
def test_backward_matches_finite_differences(ln, dual, chunk):
    x, dout, dWf = _case(1, 2, 5, 4, seed=1)

    def loss(**over):
        o, W = oracle.ttt_linear_forward(**{**x, **over}, ln=ln, dual=dual, chunk=chunk)
        return float((o * dout).sum() + (W * dWf).sum())

    g = oracle.ttt_linear_backward(**x, dout=dout, dW_final=dWf, ln=ln, dual=dual, chunk=chunk)
    h = 1e-6
    for name, key in GRADS:
        if g[key] is None:
            assert ln == "none" and name in ("gamma", "beta")
            continue
        arr = x[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            fd[idx] = (loss(**{name: a1}) - loss(**{name: a2})) / (2 * h)
        err = np.max(np.abs(fd - g[key])) / max(1e-12, np.max(np.abs(fd)))
        assert err < 1e-6, f"{name}: finite-difference mismatch {err:.2e}"


def _torch_forward(x, ln, dual, chunk, eps=oracle.EPS, silu_qk=False):
    """An independent float64 forward: LayerNorm from torch, the exact inner
    gradient by autograd, the dual form by an explicit chunk-start copy; with
    ``silu_qk`` torch's silu on keys and queries first."""
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    q, k, v, el, gl, W = t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"]
    if silu_qk:
        q, k = torch.nn.functional.silu(q), torch.nn.functional.silu(k)
    B, H, T, d = q.shape
    gam, bet = t["gamma"], t["beta"]
    outs = []
    Wc = W
    for s in range(T):
        if dual and s % chunk == 0:
            Wc = W
        P = Wc if dual else W
        z = (P @ k[:, :, s, :, None])[..., 0]
        if ln == "none":
            delta = z - v[:, :, s, :]
        else:
            zn = torch.nn.functional.layer_norm(z, (d,), eps=eps)
            pred = gam * zn + bet
            if ln == "st":
                delta = pred - v[:, :, s, :]
            else:
                zz = z if z.requires_grad else z.requires_grad_()
                lossi = 0.5 * ((gam * torch.nn.functional.layer_norm(zz, (d,), eps=eps)
                                + bet - v[:, :, s, :]) ** 2).sum()
                (delta,) = torch.autograd.grad(lossi, zz, create_graph=True)
        eta = torch.sigmoid(el[:, :, s]) / d
        W = W - eta[..., None, None] * delta[..., :, None] * k[:, :, s, None, :]
        outs.append((W @ q[:, :, s, :, None])[..., 0] * torch.sigmoid(gl[:, :, s, :]))
    return t, torch.stack(outs, dim=2), W


@pytest.mark.parametrize("ln,dual,chunk", MODES)
def test_backward_matches_autograd(ln, dual, chunk):
    x, dout, dWf = _case(2, 2, 12, 8, seed=2)
    t, out, Wf = _torch_forward(x, ln, dual, chunk)
    L = (out * torch.tensor(dout)).sum() + (Wf * torch.tensor(dWf)).sum()
    L.backward()
    g = oracle.ttt_linear_backward(**x, dout=dout, dW_final=dWf, ln=ln, dual=dual, chunk=chunk)
    for name, key in GRADS:
        if g[key] is None:
            continue
        ref = t[name].grad.numpy()
        err = np.max(np.abs(ref - g[key])) / max(1e-300, np.max(np.abs(ref)))
        assert err < 1e-10, f"{name}: autograd mismatch {err:.2e}"


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
def test_backward_eta_zero_closed_form(ln):
    x, dout, dWf = _case(1, 3, 7, 6, seed=3)
    x["eta_logit"] = np.full_like(x["eta_logit"], -np.inf)
    g = oracle.ttt_linear_backward(**x, dout=dout, dW_final=dWf, ln=ln)
    sg = 1.0 / (1.0 + np.exp(-x["gate_logit"]))
    W0 = x["W0"]
    dy = dout * sg
    y = np.einsum("bhij,bhtj->bhti", W0, x["q"])
    np.testing.assert_allclose(g["dq"], np.einsum("bhij,bhti->bhtj", W0, dy), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g["dW0"], dWf + np.einsum("bhti,bhtj->bhij", dy, x["q"]),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g["dgate_logit"], dout * y * sg * (1 - sg), rtol=1e-13, atol=1e-13)
    for key in ("dk", "dv", "deta_logit"):
        assert np.all(g[key] == 0.0), key
    if ln != "none":
        assert np.all(g["dgamma"] == 0.0) and np.all(g["dbeta"] == 0.0)


def test_ln_jacobian_derivative_finite_differences():
    rng = np.random.default_rng(4)
    d = 6
    z, gam, bet = rng.standard_normal(d), 1 + 0.3 * rng.standard_normal(d), rng.standard_normal(d)

    def jac(zz):
        _, xh, s = oracle.layer_norm(zz, gam, bet)
        return oracle.ln_jacobian(xh, s, gam)

    _, xh, s = oracle.layer_norm(z, gam, bet)
    D = oracle.ln_jacobian_derivative(xh, s, gam)
    h = 1e-6
    for p in range(d):
        zp, zm = z.copy(), z.copy()
        zp[p] += h
        zm[p] -= h
        fd = (jac(zp) - jac(zm)) / (2 * h)
        np.testing.assert_allclose(D[:, :, p], fd, rtol=1e-6, atol=1e-8)


def test_backward_without_final_state_gradient():
    x, dout, _ = _case(1, 2, 6, 4, seed=5)
    g0 = oracle.ttt_linear_backward(**x, dout=dout, dW_final=None)
    g1 = oracle.ttt_linear_backward(**x, dout=dout, dW_final=np.zeros_like(x["W0"]))
    for _, key in GRADS:
        np.testing.assert_array_equal(g0[key], g1[key])


# planted mistakes in the oracle backward (on the CPU): each must be caught
def _vjp_drop_jtj(dd, z, v, gamma, beta, ln, eps=oracle.EPS):
    dz, dv, dg, db = _REAL_VJP(dd, z, v, gamma, beta, ln, eps)
    if ln == "exact":
        _, xh, s = oracle.layer_norm(z, gamma, beta, eps)
        j = oracle.ln_jacobian(xh, s, gamma)
        dz = dz - np.matmul(np.swapaxes(j, -1, -2) @ j, dd[..., None])[..., 0]
    return dz, dv, dg, db


def _vjp_sign_dv(dd, z, v, gamma, beta, ln, eps=oracle.EPS):
    dz, dv, dg, db = _REAL_VJP(dd, z, v, gamma, beta, ln, eps)
    return dz, -dv, dg, db


def _vjp_dgamma_unscaled(dd, z, v, gamma, beta, ln, eps=oracle.EPS):
    dz, dv, dg, db = _REAL_VJP(dd, z, v, gamma, beta, ln, eps)
    return dz, dv, (None if dg is None else dg / gamma), db


_REAL_VJP = oracle.ttt_oracle.inner_grad_vector_vjp


@pytest.mark.parametrize("fake,ln", [(_vjp_drop_jtj, "exact"), (_vjp_sign_dv, "st"),
                                     (_vjp_dgamma_unscaled, "exact")])
def test_planted_backward_mistakes_are_caught(fake, ln, monkeypatch):
    monkeypatch.setattr(oracle.ttt_oracle, "inner_grad_vector_vjp", fake)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd(ln, False, 1)
