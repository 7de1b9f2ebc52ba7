"""GPU parity of training outside the matrix-core backward's reach: d = 16,
32 and 128, the dual form with any chunk length, and the vector-ALU backward
at d = 64 (TTT_FORCE_VALU), against the float64 oracle's reverse-mode
gradients.

The recording forward runs first on the GPU (the vector-ALU kernel for these
calls); its record feeds the backward.  Every element of every gradient is
compared, on several 16-token tiles plus a ragged tail.  Tolerances as for the
other backward tests: relative max error per tensor, 1e-4 for fp32 inputs and
2e-2 for bf16 inputs (the oracle sees the same bf16-rounded values).
"""
import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import make_case, make_cotangents, make_inputs

from .test_parity_backward_gpu import GRADS, TOL, assert_close, compare, cot, dev, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402


def gpu_bwd(x, dout, dWf, *, dual=False, chunk=16, silu_qk=False, force_valu=False,
            force_valu_fwd=None):
    ln = x.ln
    t = dev(x)
    gam = None if ln == "none" else t["gamma"]
    bet = None if ln == "none" else t["beta"]
    fv_fwd = force_valu if force_valu_fwd is None else force_valu_fwd
    out, Wf, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                      t["W0"], gam, bet, ln=ln, dual=dual, chunk=chunk,
                                      silu_qk=silu_qk, force_valu=fv_fwd)
    g = ttt.backward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], gam, bet, rec,
                     cot(dout), cot(dWf), ln=ln, dual=dual, chunk=chunk, silu_qk=silu_qk,
                     force_valu=force_valu)
    torch.cuda.synchronize()
    return {k: None if v is None else v.cpu().numpy() for k, v in g.items()}


def ref_bwd(x, dout, dWf, *, dual=False, chunk=16, silu_qk=False):
    return oracle.ttt_linear_backward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                      x.beta, dout, dWf, ln=x.ln, dual=dual, chunk=chunk,
                                      silu_qk=silu_qk)


def mode(ln, dual=False, force_valu=False):
    return ttt.mode_bits(ln, dual, False, False, force_valu)


@pytest.mark.parametrize("d", [16, 32, 128])
@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("bf16", [False, True])
def test_per_token_backward_other_d(d, ln, bf16):
    T = 3 * 16 + 5
    say(f"case valu backward d={d} ln={ln} bf16={bf16} T={T}")
    assert ttt.ttt_linear_backward_kernel(d, mode(ln), 1) == "bwd_valu"
    x = make_case(2, 3, T, d, seed=500 + d, ln=ln, in_bf16=bf16, random_affine=True)
    dout, dWf = make_cotangents(2, 3, T, d, seed=501 + d)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), TOL[bf16])


@pytest.mark.parametrize("d,chunk", [(16, 1), (16, 5), (16, 16), (16, 37), (32, 8), (64, 5),
                                     (64, 8), (64, 32), (64, 48), (128, 7), (128, 16)])
@pytest.mark.parametrize("ln", ["st", "exact"])
def test_dual_backward_any_chunk(d, chunk, ln):
    T = 70
    say(f"case valu dual backward d={d} chunk={chunk} ln={ln} T={T}")
    assert ttt.ttt_linear_backward_kernel(d, mode(ln, True), chunk) == "bwd_valu"
    x = make_case(2, 2, T, d, seed=510 + chunk, ln=ln, dual=True, chunk=chunk,
                  random_affine=True)
    dout, dWf = make_cotangents(2, 2, T, d, seed=511 + chunk)
    compare(gpu_bwd(x, dout, dWf, dual=True, chunk=chunk),
            ref_bwd(x, dout, dWf, dual=True, chunk=chunk), 1e-4)


@pytest.mark.parametrize("chunk", [3, 100])
def test_dual_backward_bf16_no_ln(chunk):
    say(f"case valu dual backward bf16 none chunk={chunk}")
    x = make_case(2, 2, 90, 32, seed=520 + chunk, ln="none", dual=True, chunk=chunk,
                  in_bf16=True)
    dout, dWf = make_cotangents(2, 2, 90, 32, seed=521)
    compare(gpu_bwd(x, dout, dWf, dual=True, chunk=chunk),
            ref_bwd(x, dout, dWf, dual=True, chunk=chunk), TOL[True])


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("bf16", [False, True])
def test_forced_vector_alu_backward_at_d64(ln, bf16):
    # the kernel the matrix-core backward replaces, on the same record format
    say(f"case valu backward d=64 forced ln={ln} bf16={bf16}")
    assert ttt.ttt_linear_backward_kernel(64, mode(ln, force_valu=True), 1) == "bwd_valu"
    x = make_case(2, 3, 53, 64, seed=530, ln=ln, in_bf16=bf16, random_affine=True)
    dout, dWf = make_cotangents(2, 3, 53, 64, seed=531)
    compare(gpu_bwd(x, dout, dWf, force_valu=True), ref_bwd(x, dout, dWf), TOL[bf16])


@pytest.mark.parametrize("dual", [False, True])
def test_records_of_either_forward_serve_either_backward(dual):
    # the matrix-core forward's record into the vector-ALU backward, and the
    # vector-ALU forward's record into the matrix-core backward
    say(f"case mixed record/backward kernels dual={dual}")
    x = make_case(2, 2, 45, 64, seed=540, ln="exact", dual=dual, chunk=16, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 45, 64, seed=541)
    r = ref_bwd(x, dout, dWf, dual=dual)
    compare(gpu_bwd(x, dout, dWf, dual=dual, force_valu=True, force_valu_fwd=False), r, 1e-4)
    compare(gpu_bwd(x, dout, dWf, dual=dual, force_valu=False, force_valu_fwd=True), r, 1e-4)


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 33])
def test_short_and_ragged_backward_d32(T):
    say(f"case valu backward d=32 T={T}")
    x = make_case(2, 2, T, 32, seed=550 + T, ln="st", random_affine=True)
    dout, dWf = make_cotangents(2, 2, T, 32, seed=551 + T)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), 1e-4)
    compare(gpu_bwd(x, dout, dWf, dual=True, chunk=5),
            ref_bwd(x, dout, dWf, dual=True, chunk=5), 1e-4)


@pytest.mark.parametrize("d,dual,chunk", [(16, False, 1), (128, True, 8), (64, True, 12)])
def test_silu_backward_vector_alu(d, dual, chunk):
    say(f"case valu backward silu d={d} dual={dual} chunk={chunk}")
    x = make_case(2, 2, 50, d, seed=560 + d, in_bf16=True, dual=dual, chunk=chunk,
                  random_affine=True)
    dout, dWf = make_cotangents(2, 2, 50, d, seed=561)
    compare(gpu_bwd(x, dout, dWf, dual=dual, chunk=chunk, silu_qk=True),
            ref_bwd(x, dout, dWf, dual=dual, chunk=chunk, silu_qk=True), TOL[True])


def test_empty_sequence_d16():
    say("case valu backward T=0 d=16")
    x = make_case(2, 3, 0, 16, seed=570, random_affine=True)
    dout, dWf = make_cotangents(2, 3, 0, 16, seed=571)
    g = gpu_bwd(x, dout, dWf, dual=True, chunk=5)
    assert np.array_equal(g["dW0"], dWf)
    assert np.all(g["dgamma"] == 0) and np.all(g["dbeta"] == 0)


def test_eta_zero_closed_form_d32_dual():
    # eta_logit = -inf: W stays W0, so dk = dv = d eta = 0 exactly,
    # dq_t = W0^T dy_t and dW0 = dW_final + sum_t dy_t q_t^T
    say("case valu backward eta=-inf d=32 dual chunk 6")
    x = make_case(2, 2, 50, 32, seed=580, random_affine=True, dual=True, chunk=6)
    x.eta_logit[:] = -np.inf
    dout, dWf = make_cotangents(2, 2, 50, 32, seed=581)
    g = gpu_bwd(x, dout, dWf, dual=True, chunk=6)
    for key in ("dk", "dv", "deta_logit", "dgamma", "dbeta"):
        assert np.all(g[key] == 0.0), key
    sg = 1.0 / (1.0 + np.exp(-x.gate_logit.astype(np.float64)))
    dy = dout * sg
    W0 = x.W0.astype(np.float64)
    assert_close(g["dq"], np.einsum("bhij,bhti->bhtj", W0, dy), 1e-5, "dq")
    assert_close(g["dW0"], dWf + np.einsum("bhti,bhtj->bhij", dy, x.q.astype(np.float64)), 1e-5,
                 "dW0")


@pytest.mark.parametrize("d,dual,chunk,force", [(16, False, 1, False), (32, True, 5, False),
                                                (128, True, 16, False), (64, True, 8, False),
                                                (64, False, 1, True)])
def test_vector_alu_record_forward_matches_plain_forward_bitwise(d, dual, chunk, force):
    say(f"case valu forward_record == forward d={d} dual={dual} chunk={chunk}")
    for ln, bf16 in (("st", True), ("exact", False), ("none", False)):
        x = make_case(2, 3, 70, d, seed=590, ln=ln, in_bf16=bf16, random_affine=True)
        t = dev(x)
        gam = None if ln == "none" else t["gamma"]
        bet = None if ln == "none" else t["beta"]
        o1, W1 = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                             gam, bet, ln=ln, dual=dual, chunk=chunk, force_valu=force)
        o2, W2, _ = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"],
                                       t["gate_logit"], t["W0"], gam, bet, ln=ln, dual=dual,
                                       chunk=chunk, force_valu=force)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(W1, W2), (ln, bf16)


def test_autograd_d16_dual_chunk5():
    say("case valu autograd d=16 dual chunk 5")
    x = make_case(2, 2, 41, 16, seed=600, dual=True, chunk=5, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 41, 16, seed=601)
    t = dev(x)
    leaves = {k: v.clone().requires_grad_() for k, v in t.items()}
    out, Wf = ttt.ttt_linear(*[leaves[k] for k in ("q", "k", "v", "eta_logit", "gate_logit",
                                                   "W0", "gamma", "beta")], ln="st", dual=True,
                             chunk=5)
    ((out * cot(dout)).sum() + (Wf * cot(dWf)).sum()).backward()
    r = ref_bwd(x, dout, dWf, dual=True, chunk=5)
    names = dict(q="dq", k="dk", v="dv", eta_logit="deta_logit", gate_logit="dgate_logit",
                 W0="dW0", gamma="dgamma", beta="dbeta")
    for leaf, key in names.items():
        assert_close(leaves[leaf].grad.cpu().numpy(), r[key], 1e-4, f"autograd {key}")


def test_vector_alu_backward_repeatable():
    say("case valu backward repeat")
    x = make_case(2, 2, 45, 128, seed=610, ln="exact", dual=True, chunk=9, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 45, 128, seed=611)
    g1 = gpu_bwd(x, dout, dWf, dual=True, chunk=9)
    g2 = gpu_bwd(x, dout, dWf, dual=True, chunk=9)
    for key in GRADS:
        assert np.array_equal(g1[key], g2[key]), key


def test_full_size_tiny_d16_workload():
    # the d = 16 workload at its full size (B=1, H=2, T=64, fp32): every scan
    say("case valu backward full size tiny_d16_fp32")
    x = make_inputs("tiny_d16_fp32")
    B, H, T, d = x.q.shape
    dout, dWf = make_cotangents(B, H, T, d, seed=620)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), 1e-4)
    compare(gpu_bwd(x, dout, dWf, dual=True, chunk=8),
            ref_bwd(x, dout, dWf, dual=True, chunk=8), 1e-4)


def test_long_d128_dual_sampled():
    # a longer d = 128 scan (many tiles, chunks that straddle tiles), two scans
    say("case valu backward d=128 T=1000 dual chunk 24")
    x = make_case(1, 2, 1000, 128, seed=630, ln="st", dual=True, chunk=24, random_affine=True,
                  l2norm_qkv=True, eta_mean=-1.0)
    dout, dWf = make_cotangents(1, 2, 1000, 128, seed=631)
    compare(gpu_bwd(x, dout, dWf, dual=True, chunk=24),
            ref_bwd(x, dout, dWf, dual=True, chunk=24), 1e-4)
