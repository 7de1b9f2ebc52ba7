"""Pins of the oracle's input projections (``oracle.input_projections``)
against things fixed independently of its matrix product: a brute-force
loop, weight rows that select single coordinates of x (so the split into
q, k, v, gate, eta and the head order show directly), the bias alone, and
linearity in x."""
import numpy as np
import pytest

import oracle


def brute(x, w, b):
    B, T, hidden = x.shape
    H, R, _ = w.shape
    d = (R - 1) // 4
    out = {n: np.zeros((B, H, T, d)) for n in ("q", "k", "v", "gate")}
    eta = np.zeros((B, H, T))
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                for r in range(R):
                    acc = 0.0 if b is None else float(b[h, r])
                    for j in range(hidden):
                        acc += float(x[bb, t, j]) * float(w[h, r, j])
                    if r == 4 * d:
                        eta[bb, h, t] = acc
                    else:
                        out[("q", "k", "v", "gate")[r // d]][bb, h, t, r % d] = acc
    return out["q"], out["k"], out["v"], eta, out["gate"]


@pytest.mark.parametrize("with_bias", [False, True])
def test_matches_brute_force_loop(with_bias):
    rng = np.random.default_rng(0)
    B, T, hidden, H, d = 2, 3, 5, 2, 2
    x = rng.standard_normal((B, T, hidden))
    w = rng.standard_normal((H, 4 * d + 1, hidden))
    b = rng.standard_normal((H, 4 * d + 1)) if with_bias else None
    got = oracle.input_projections(x, w, b)
    ref = brute(x, w, b)
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        np.testing.assert_allclose(g, r, rtol=1e-13, atol=1e-13)


def test_one_hot_rows_pick_coordinates_in_the_stated_order():
    # row r of head h selects coordinate sel[h, r] of x: the outputs must be
    # exactly those coordinates, in the order q, k, v, gate, eta
    B, T, H, d = 2, 4, 3, 2
    R = 4 * d + 1
    hidden = H * R
    rng = np.random.default_rng(1)
    x = rng.standard_normal((B, T, hidden))
    sel = rng.permutation(hidden).reshape(H, R)
    w = np.zeros((H, R, hidden))
    for h in range(H):
        for r in range(R):
            w[h, r, sel[h, r]] = 1.0
    q, k, v, eta, gate = oracle.input_projections(x, w)
    for h in range(H):
        for i in range(d):
            assert np.array_equal(q[:, h, :, i], x[:, :, sel[h, i]])
            assert np.array_equal(k[:, h, :, i], x[:, :, sel[h, d + i]])
            assert np.array_equal(v[:, h, :, i], x[:, :, sel[h, 2 * d + i]])
            assert np.array_equal(gate[:, h, :, i], x[:, :, sel[h, 3 * d + i]])
        assert np.array_equal(eta[:, h, :], x[:, :, sel[h, 4 * d]])


def test_bias_alone():
    B, T, hidden, H, d = 1, 5, 7, 2, 3
    b = np.arange(H * (4 * d + 1), dtype=np.float64).reshape(H, 4 * d + 1)
    q, k, v, eta, gate = oracle.input_projections(np.ones((B, T, hidden)),
                                                  np.zeros((H, 4 * d + 1, hidden)), b)
    for h in range(H):
        assert np.all(q[:, h] == b[h, :d]) and np.all(k[:, h] == b[h, d:2 * d])
        assert np.all(v[:, h] == b[h, 2 * d:3 * d]) and np.all(gate[:, h] == b[h, 3 * d:4 * d])
        assert np.all(eta[:, h] == b[h, 4 * d])


def test_linear_in_x():
    rng = np.random.default_rng(2)
    x1, x2 = rng.standard_normal((2, 2, 6, 8))
    w = rng.standard_normal((3, 9, 8))
    a = oracle.input_projections(2.5 * x1 - 0.5 * x2, w)
    p1 = oracle.input_projections(x1, w)
    p2 = oracle.input_projections(x2, w)
    for got, u, v in zip(a, p1, p2):
        np.testing.assert_allclose(got, 2.5 * u - 0.5 * v, rtol=1e-12, atol=1e-12)


def test_rejects_a_stack_that_is_not_4d_plus_1_rows():
    with pytest.raises(ValueError):
        oracle.input_projections(np.zeros((1, 2, 4)), np.zeros((1, 8, 4)))
