"""The seeded input generator: determinism, bf16 rounding and the recipe."""
import numpy as np
import torch

from test_rnn_layer_ttt_amd.inputs import WORKLOADS, make_case, make_inputs, round_to_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e-39,
                                  65504.0, -1e30], np.float32)])
    got = round_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_seeded_and_deterministic():
    a = make_case(2, 3, 17, 8, seed=5, in_bf16=True, random_affine=True)
    b = make_case(2, 3, 17, 8, seed=5, in_bf16=True, random_affine=True)
    c = make_case(2, 3, 17, 8, seed=6, in_bf16=True, random_affine=True)
    for f in ("q", "k", "v", "eta_logit", "gate_logit", "W0", "gamma", "beta"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert getattr(a, f).dtype == np.float32 and getattr(a, f).flags.c_contiguous
    assert not np.array_equal(a.q, c.q)
    # bf16 inputs hold exactly representable values
    assert np.array_equal(round_to_bf16(a.q), a.q)


def test_recipe_statistics():
    x = make_case(4, 4, 512, 64, seed=1, l2norm_qkv=True, random_affine=True, eta_mean=-1.0)
    assert abs(x.W0.std() - 0.02) < 0.001
    assert np.allclose(np.linalg.norm(x.k.astype(np.float64), axis=-1), 8.0, rtol=1e-6)
    assert abs(x.eta_logit.mean() + 1.0) < 0.05
    assert abs(x.gamma.mean() - 1.0) < 0.05 and abs(x.beta.mean()) < 0.05


def test_workload_table_shapes():
    assert WORKLOADS["h1024_T4096_bf16"]["B"] * WORKLOADS["h1024_T4096_bf16"]["H"] == 256
    x = make_inputs("tiny_d16_fp32")
    assert x.q.shape == (1, 2, 64, 16) and x.eta_logit.shape == (1, 2, 64)
    assert x.W0.shape == (1, 2, 16, 16) and x.gamma.shape == (2, 16)
    s = x.subset([(0, 1), (0, 0)])
    assert s.q.shape == (1, 2, 64, 16) and np.array_equal(s.q[0, 0], x.q[0, 1])
    assert np.array_equal(s.gamma[0], x.gamma[1])
