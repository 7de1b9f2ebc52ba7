"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Every mutation below is a mistake one could make while writing the oracle
from the pages; each must make at least one pin in ``test_oracle`` fail.
"""
import numpy as np
import pytest

import oracle.ttt_oracle as ora
import tests.test_oracle as pins


def _layer_norm_unbiased(z, gamma, beta, eps=ora.EPS):
    d = z.shape[-1]
    mu = z.mean(-1, keepdims=True)
    var = ((z - mu) ** 2).sum(-1, keepdims=True) / (d - 1)
    s = np.sqrt(var + eps)
    return gamma * (z - mu) / s + beta, (z - mu) / s, s


def _layer_norm_eps_outside(z, gamma, beta, eps=ora.EPS):
    mu = z.mean(-1, keepdims=True)
    s = np.sqrt(((z - mu) ** 2).mean(-1, keepdims=True)) + eps
    return gamma * (z - mu) / s + beta, (z - mu) / s, s


def _grad_sign_flipped(z, v, gamma, beta, ln, eps=ora.EPS):
    return -_orig_grad(z, v, gamma, beta, ln, eps)


def _grad_jacobian_untransposed(z, v, gamma, beta, ln, eps=ora.EPS):
    if ln != ora.LN_EXACT:
        return _orig_grad(z, v, gamma, beta, ln, eps)
    pred, xhat, s = ora.layer_norm(z, gamma, beta, eps)
    jac = ora.ln_jacobian(xhat, s, gamma)
    return np.matmul(jac, (pred - v)[..., None])[..., 0]


def _jacobian_drop_mean_term(xhat, s, gamma):
    d = xhat.shape[-1]
    core = np.eye(d) - xhat[..., :, None] * xhat[..., None, :] / d
    return (gamma[..., :, None] / s[..., None]) * core


_orig_grad = ora.inner_grad_vector
_orig_forward = ora.ttt_linear_forward


def _forward_transposed_W(q, k, v, eta_logit, gate_logit, W0, *a, **kw):
    W0 = np.swapaxes(np.asarray(W0), -1, -2)
    out, W = _orig_forward(q, k, v, eta_logit, gate_logit, W0, *a, **kw)
    return out, np.swapaxes(W, -1, -2)


MUTATIONS = {
    "unbiased_variance": ("layer_norm", _layer_norm_unbiased),
    "eps_outside_sqrt": ("layer_norm", _layer_norm_eps_outside),
    "gradient_sign": ("inner_grad_vector", _grad_sign_flipped),
    "jacobian_not_transposed": ("inner_grad_vector", _grad_jacobian_untransposed),
    "jacobian_missing_mean_term": ("ln_jacobian", _jacobian_drop_mean_term),
}

PIN_SUITE = [
    (pins.test_layer_norm_matches_torch, {}),
    (pins.test_hand_worked_example, {}),
    (pins.test_scan_equals_autograd_inner_steps, {"ln": "st"}),
    (pins.test_scan_equals_autograd_inner_steps, {"ln": "exact"}),
    (pins.test_exact_gradient_finite_differences, {}),
    (pins.test_delta_rule_unrolled_product, {}),
]


def _some_pin_fails():
    for fn, kw in PIN_SUITE:
        try:
            fn(**kw)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(ora, attr, fake)
    monkeypatch.setattr(pins.oracle, attr, fake, raising=False)
    assert _some_pin_fails(), f"mutation {name} slipped through every pin"


def test_transposed_weight_is_caught(monkeypatch):
    monkeypatch.setattr(pins.oracle, "ttt_linear_forward", _forward_transposed_W)
    assert _some_pin_fails()


def test_unmutated_oracle_passes_suite():
    assert not _some_pin_fails()
