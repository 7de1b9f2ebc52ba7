"""Pins of the oracle's `:mlp` variant ("Edifice.Recurrent.TTT", Options,
`:variant`: SiLU on keys and queries before the inner model).

The activation is checked against torch's silu and its derivative against
autograd; the variant's forward against the plain scan fed torch-activated
keys and queries; its backward against central finite differences and
against autograd through an independent torch forward."""
import numpy as np
import pytest

import oracle

from .test_oracle_backward import GRADS, _case, _torch_forward

torch = pytest.importorskip("torch")


def test_silu_and_its_derivative_match_torch():
    x = np.concatenate([np.linspace(-40, 40, 401), [-1e4, 1e4, 0.0]])
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.silu(t)
    y.sum().backward()
    np.testing.assert_allclose(oracle.silu(x), y.detach().numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.silu_grad(x), t.grad.numpy(), rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("ln,dual,chunk", [("st", False, 1), ("exact", False, 1),
                                           ("none", True, 3)])
def test_variant_is_the_scan_on_activated_keys_and_queries(ln, dual, chunk):
    x, _, _ = _case(2, 2, 9, 6, seed=21)
    act = lambda a: torch.nn.functional.silu(torch.tensor(a, dtype=torch.float64)).numpy()
    o1, W1 = oracle.ttt_linear_forward(**x, ln=ln, dual=dual, chunk=chunk, silu_qk=True)
    o2, W2 = oracle.ttt_linear_forward(**{**x, "q": act(x["q"]), "k": act(x["k"])}, ln=ln,
                                       dual=dual, chunk=chunk)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(W1, W2, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
def test_variant_backward_matches_finite_differences(ln):
    x, dout, dWf = _case(1, 2, 5, 4, seed=22)

    def loss(**over):
        o, W = oracle.ttt_linear_forward(**{**x, **over}, ln=ln, silu_qk=True)
        return float((o * dout).sum() + (W * dWf).sum())

    g = oracle.ttt_linear_backward(**x, dout=dout, dW_final=dWf, ln=ln, silu_qk=True)
    h = 1e-6
    for name, key in GRADS:
        if g[key] is None:
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


@pytest.mark.parametrize("ln", ["st", "exact"])
def test_variant_backward_matches_autograd(ln):
    x, dout, dWf = _case(2, 2, 10, 8, seed=23)
    t, out, Wf = _torch_forward({**x}, ln, False, 1, silu_qk=True)
    ((out * torch.tensor(dout)).sum() + (Wf * torch.tensor(dWf)).sum()).backward()
    g = oracle.ttt_linear_backward(**x, dout=dout, dW_final=dWf, ln=ln, silu_qk=True)
    for name, key in GRADS:
        if g[key] is None:
            continue
        ref = t[name].grad.numpy()
        err = np.max(np.abs(ref - g[key])) / max(1e-300, np.max(np.abs(ref)))
        assert err < 1e-10, f"{name}: autograd mismatch {err:.2e}"
