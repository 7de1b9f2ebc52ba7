"""GPU parity of the backward pass (through the C ABI) against the float64
oracle's reverse-mode gradients.

The recording forward runs first on the GPU; its record feeds the backward.
Small cases compare every element of every gradient; the full-size workloads
run exactly as the benchmark launches them and are compared on sampled
scans (all batches of one head, so that dgamma and dbeta, which sum over the
batch, can be compared as well).  Tolerances: relative max error per tensor,
1e-4 for fp32 inputs and 2e-2 for bf16 inputs (the oracle sees the same
bf16-rounded values), as for the forward.
"""
import sys

import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import (make_case, make_cotangents, make_inputs,
                                           make_update_mask)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402

TOL = {False: 1e-4, True: 2e-2}
GRADS = ("dq", "dk", "dv", "dgate_logit", "deta_logit", "dW0", "dgamma", "dbeta")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x):
    dt = torch.bfloat16 if x.in_bf16 else torch.float32
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(q=f(x.q), k=f(x.k), v=f(x.v), eta_logit=f(x.eta_logit),
                gate_logit=f(x.gate_logit), W0=g(x.W0), gamma=g(x.gamma), beta=g(x.beta))


def cot(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_bwd(x, dout, dWf, ln=None, dual=False, silu_qk=False):
    ln = x.ln if ln is None else ln
    t = dev(x)
    gam = None if ln == "none" else t["gamma"]
    bet = None if ln == "none" else t["beta"]
    out, Wf, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                      t["W0"], gam, bet, ln=ln, dual=dual, silu_qk=silu_qk)
    g = ttt.backward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], gam, bet, rec,
                     cot(dout), cot(dWf), ln=ln, dual=dual, silu_qk=silu_qk)
    torch.cuda.synchronize()
    return {k: None if v is None else v.cpu().numpy() for k, v in g.items()}


def ref_bwd(x, dout, dWf, ln=None, dual=False, silu_qk=False):
    return oracle.ttt_linear_backward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                      x.beta, dout, dWf, ln=x.ln if ln is None else ln,
                                      dual=dual, chunk=16, silu_qk=silu_qk)


def assert_close(got, ref, tol, what):
    err = oracle.rel_max_err(got, ref)
    say(f"    {what}: rel max err {err:.3g} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: rel max err {err:.3g} > {tol:g}"


def compare(g, r, tol, keys=GRADS):
    for key in keys:
        if r[key] is None:
            assert g[key] is None, key
            continue
        assert_close(g[key], r[key], tol, key)


# ---------------------------------------------------------------------------
# small cases: every gradient element, several tiles plus a ragged tail
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("bf16", [False, True])
def test_small_backward_parity(ln, bf16):
    T = 3 * 16 + 5
    say(f"case backward ln={ln} bf16={bf16} T={T}")
    x = make_case(2, 3, T, 64, seed=300 + T, ln=ln, in_bf16=bf16, random_affine=True)
    dout, dWf = make_cotangents(2, 3, T, 64, seed=301)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), TOL[bf16])


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 32, 33, 100])
@pytest.mark.parametrize("ln", ["st", "exact"])
def test_short_and_ragged_backward(T, ln):
    say(f"case backward T={T} ln={ln}")
    x = make_case(2, 2, T, 64, seed=310 + T, ln=ln, random_affine=True)
    dout, dWf = make_cotangents(2, 2, T, 64, seed=311 + T)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), 1e-4)


def test_backward_unit_norm_inputs_and_negative_eta():
    # the distributions of the hidden-256 and exact-LayerNorm workloads
    say("case backward l2norm, eta_mean=-1, exact")
    x = make_case(3, 2, 90, 64, seed=320, ln="exact", l2norm_qkv=True, random_affine=True,
                  eta_mean=-1.0)
    dout, dWf = make_cotangents(3, 2, 90, 64, seed=321)
    compare(gpu_bwd(x, dout, dWf), ref_bwd(x, dout, dWf), 1e-4)


def test_backward_without_state_gradient():
    say("case backward dW_final=None")
    x = make_case(2, 2, 40, 64, seed=330, random_affine=True)
    dout, _ = make_cotangents(2, 2, 40, 64, seed=331, with_state=False)
    compare(gpu_bwd(x, dout, None), ref_bwd(x, dout, None), 1e-4)


def test_backward_empty_sequence():
    say("case backward T=0")
    x = make_case(2, 3, 0, 64, seed=340, random_affine=True)
    dout, dWf = make_cotangents(2, 3, 0, 64, seed=341)
    g = gpu_bwd(x, dout, dWf)
    assert np.array_equal(g["dW0"], dWf)
    assert np.all(g["dgamma"] == 0) and np.all(g["dbeta"] == 0)
    for key in ("dq", "dk", "dv", "dgate_logit", "deta_logit"):
        assert g[key].size == 0


def test_backward_eta_zero_closed_form():
    # eta_logit = -inf: W stays W0, so dk = dv = d eta = 0 exactly and
    # dq_t = W0^T dy_t, dW0 = dW_final + sum_t dy_t q_t^T
    say("case backward eta=-inf")
    x = make_case(2, 2, 50, 64, seed=350, random_affine=True)
    x.eta_logit[:] = -np.inf
    dout, dWf = make_cotangents(2, 2, 50, 64, seed=351)
    g = gpu_bwd(x, dout, dWf)
    for key in ("dk", "dv", "deta_logit", "dgamma", "dbeta"):
        assert np.all(g[key] == 0.0), key
    sg = 1.0 / (1.0 + np.exp(-x.gate_logit.astype(np.float64)))
    dy = dout * sg
    W0 = x.W0.astype(np.float64)
    assert_close(g["dq"], np.einsum("bhij,bhti->bhtj", W0, dy), 1e-5, "dq")
    assert_close(g["dW0"], dWf + np.einsum("bhti,bhtj->bhij", dy, x.q.astype(np.float64)), 1e-5,
                 "dW0")


def test_record_forward_matches_plain_forward_bitwise():
    say("case forward_record == forward")
    for ln, bf16 in (("st", True), ("exact", False), ("none", False)):
        x = make_case(2, 3, 70, 64, seed=360, ln=ln, in_bf16=bf16, random_affine=True)
        t = dev(x)
        gam = None if ln == "none" else t["gamma"]
        bet = None if ln == "none" else t["beta"]
        o1, W1 = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                             gam, bet, ln=ln)
        o2, W2, _ = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"],
                                       t["gate_logit"], t["W0"], gam, bet, ln=ln)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(W1, W2), (ln, bf16)


def test_backward_repeatable_and_in_place_state_gradient():
    # two calls on one record give identical bits; dW0 may be dW_final itself
    say("case backward repeat + in place")
    x = make_case(2, 2, 45, 64, seed=370, ln="exact", random_affine=True)
    dout, dWf = make_cotangents(2, 2, 45, 64, seed=371)
    t = dev(x)
    _, _, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                   t["W0"], t["gamma"], t["beta"], ln="exact")
    args = (t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["gamma"], t["beta"], rec)
    g1 = ttt.backward(*args, cot(dout), cot(dWf), ln="exact")
    g2 = ttt.backward(*args, cot(dout), cot(dWf), ln="exact")
    torch.cuda.synchronize()
    for key in GRADS:
        assert torch.equal(g1[key], g2[key]), key
    # in place through the raw entry point: dW0 == dW_final
    B, H, T, d = x.q.shape
    dW = cot(dWf).clone()
    out = {k: torch.empty_like(v) for k, v in g1.items()}
    p = lambda a: a.data_ptr()
    st, nws = ttt.ttt_linear_backward_workspace_bytes(B, H, d, ttt.mode_bits("exact"))
    assert st == ttt.TTT_OK and nws == B * H * 2 * d * 4
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    st = ttt.ttt_linear_backward(
        p(t["q"]), p(t["k"]), p(t["v"]), p(t["eta_logit"]), p(t["gate_logit"]), p(t["gamma"]),
        p(t["beta"]), p(rec), rec.numel(), p(ws), nws, p(cot(dout)), p(dW), p(out["dq"]),
        p(out["dk"]),
        p(out["dv"]), p(out["deta_logit"]), p(out["dgate_logit"]), p(dW), p(out["dgamma"]),
        p(out["dbeta"]), B, H, T, d, ttt.mode_bits("exact"), 1,
        torch.cuda.current_stream().cuda_stream)
    assert st == ttt.TTT_OK
    torch.cuda.synchronize()
    assert torch.equal(dW, g1["dW0"])


def test_concurrent_backward_calls_share_one_record():
    # the record is read-only: two backward calls on one record, on two streams
    # at once (each with its own workspace), give the bits of a lone call
    say("case concurrent backward on one record")
    x = make_case(4, 4, 300, 64, seed=372, ln="st", random_affine=True)
    dout, dWf = make_cotangents(4, 4, 300, 64, seed=373)
    t = dev(x)
    _, _, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                   t["W0"], t["gamma"], t["beta"], ln="st")
    args = (t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["gamma"], t["beta"], rec)
    ref = ttt.backward(*args, cot(dout), cot(dWf), ln="st")
    torch.cuda.synchronize()
    before = rec.clone()
    d_o, d_w = cot(dout), cot(dWf)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        g1 = ttt.backward(*args, d_o, d_w, ln="st", stream=s1)
    with torch.cuda.stream(s2):
        g2 = ttt.backward(*args, d_o, d_w, ln="st", stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(rec, before)
    for key in GRADS:
        assert torch.equal(g1[key], ref[key]) and torch.equal(g2[key], ref[key]), key


def test_autograd_function_matches_backward():
    say("case autograd")
    x = make_case(2, 2, 33, 64, seed=380, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 33, 64, seed=381)
    t = dev(x)
    leaves = {k: v.clone().requires_grad_() for k, v in t.items()}
    out, Wf = ttt.ttt_linear(*[leaves[k] for k in ("q", "k", "v", "eta_logit", "gate_logit",
                                                   "W0", "gamma", "beta")], ln="st")
    ((out * cot(dout)).sum() + (Wf * cot(dWf)).sum()).backward()
    r = ref_bwd(x, dout, dWf)
    names = dict(q="dq", k="dk", v="dv", eta_logit="deta_logit", gate_logit="dgate_logit",
                 W0="dW0", gamma="dgamma", beta="dbeta")
    for leaf, key in names.items():
        assert_close(leaves[leaf].grad.cpu().numpy(), r[key], 1e-4, f"autograd {key}")


# ---------------------------------------------------------------------------
# full-size workloads, sampled: all batches of one head
# ---------------------------------------------------------------------------
def _sampled(x, dout, dWf, head):
    """The scans of one head over all batches, stacked as B=1 (oracle inputs)."""
    B = x.q.shape[0]
    pairs = [(b, head) for b in range(B)]
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    cut = lambda a: np.ascontiguousarray(a[bs, hs][None])
    return x.subset(pairs), cut(dout), cut(dWf), (bs, hs)


@pytest.mark.parametrize("workload,head", [("h1024_T4096_bf16", 5), ("h256_T2048_fp32", 3)])
def test_full_size_backward_sampled(workload, head):
    say(f"case backward full size {workload} head {head}")
    x = make_inputs(workload)
    B, H, T, d = x.q.shape
    dout, dWf = make_cotangents(B, H, T, d, seed=390)
    g = gpu_bwd(x, dout, dWf)
    xs, ds, dWs, (bs, hs) = _sampled(x, dout, dWf, head)
    r = ref_bwd(xs, ds, dWs)
    tol = TOL[x.in_bf16]
    per_scan(g, r, bs, hs, ("dq", "dk", "dv", "dgate_logit", "deta_logit", "dW0"), tol)
    assert_close(g["dgamma"][head], r["dgamma"].sum(axis=0), tol, "dgamma")
    assert_close(g["dbeta"][head], r["dbeta"].sum(axis=0), tol, "dbeta")


def per_scan(g, r, bs, hs, keys, tol):
    """Every sampled scan on its own (its error against its own largest
    value), so that one scan's small gradients cannot hide behind another's."""
    for key in keys:
        for n, (b, h) in enumerate(zip(bs, hs)):
            assert_close(g[key][b, h], r[key][0, n], tol, f"{key}[{b},{h}]")


def test_full_size_exact_backward_tail():
    # hidden 2048, T = 16384, exact LayerNorm gradient.  The oracle's exact
    # backward is too slow for the whole sequence, but the gradients with
    # respect to the last L tokens' inputs depend only on W before them and on
    # those tokens: the oracle runs its forward to T - L, then its backward
    # over the last L tokens from that W.
    workload, head, L = "h2048_T16384_exact_fp32", 17, 512
    say(f"case backward full size {workload} head {head}, last {L} tokens")
    x = make_inputs(workload)
    B, H, T, d = x.q.shape
    dout, dWf = make_cotangents(B, H, T, d, seed=391)
    g = gpu_bwd(x, dout, dWf)
    xs, ds, dWs, (bs, hs) = _sampled(x, dout, dWf, head)
    head_part = lambda a: a[:, :, :T - L]
    tail = lambda a: np.ascontiguousarray(a[:, :, T - L:])
    _, Wmid = oracle.ttt_linear_forward(head_part(xs.q), head_part(xs.k), head_part(xs.v),
                                        head_part(xs.eta_logit), head_part(xs.gate_logit),
                                        xs.W0, xs.gamma, xs.beta, ln="exact")
    r = oracle.ttt_linear_backward(tail(xs.q), tail(xs.k), tail(xs.v), tail(xs.eta_logit),
                                   tail(xs.gate_logit), Wmid, xs.gamma, xs.beta, tail(ds), dWs,
                                   ln="exact")
    for key in ("dq", "dk", "dv", "dgate_logit", "deta_logit"):
        assert_close(tail(g[key][bs, hs][None]), r[key], 1e-4, key)


# ---------------------------------------------------------------------------
# the dual form: chunks of 16 tokens (the tiles), every z of a chunk at the
# chunk's first W
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("bf16", [False, True])
def test_dual_small_backward_parity(ln, bf16):
    T = 3 * 16 + 5
    say(f"case dual backward ln={ln} bf16={bf16} T={T}")
    x = make_case(2, 3, T, 64, seed=400 + T, ln=ln, dual=True, chunk=16, in_bf16=bf16,
                  random_affine=True)
    dout, dWf = make_cotangents(2, 3, T, 64, seed=401)
    compare(gpu_bwd(x, dout, dWf, dual=True), ref_bwd(x, dout, dWf, dual=True), TOL[bf16])


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 100])
def test_dual_short_and_ragged_backward(T):
    say(f"case dual backward T={T}")
    x = make_case(2, 2, T, 64, seed=410 + T, dual=True, chunk=16, random_affine=True)
    dout, dWf = make_cotangents(2, 2, T, 64, seed=411 + T)
    compare(gpu_bwd(x, dout, dWf, dual=True), ref_bwd(x, dout, dWf, dual=True), 1e-4)


def test_dual_backward_differs_from_per_token():
    # the two forms' gradients are not interchangeable: the per-token backward
    # on a dual record would be a silent error, so the forms must differ here
    say("case dual vs per-token gradients")
    x = make_case(1, 2, 40, 64, seed=420, dual=True, chunk=16, random_affine=True)
    dout, dWf = make_cotangents(1, 2, 40, 64, seed=421)
    g = gpu_bwd(x, dout, dWf, dual=True)
    r_tok = ref_bwd(x, dout, dWf, dual=False)
    assert oracle.rel_max_err(g["dk"], r_tok["dk"]) > 1e-2


def test_dual_record_forward_matches_plain_forward_bitwise():
    say("case dual forward_record == forward")
    for ln, bf16 in (("st", True), ("exact", False), ("none", False)):
        x = make_case(2, 3, 70, 64, seed=430, ln=ln, dual=True, chunk=16, in_bf16=bf16,
                      random_affine=True)
        t = dev(x)
        gam = None if ln == "none" else t["gamma"]
        bet = None if ln == "none" else t["beta"]
        o1, W1 = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                             gam, bet, ln=ln, dual=True, chunk=16)
        o2, W2, _ = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"],
                                       t["gate_logit"], t["W0"], gam, bet, ln=ln, dual=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(W1, W2), (ln, bf16)


def test_dual_skipped_chunks_as_minus_inf_step_size():
    # a chunk the masked forward skips trains as eta_logit = -inf on its
    # tokens: the recording forward then equals the masked forward bit for bit,
    # and the gradients match the oracle's, with d eta_logit = 0 on those tokens
    say("case dual backward, skipped chunks")
    B, H, T = 2, 3, 90
    x = make_case(B, H, T, 64, seed=440, dual=True, chunk=16, in_bf16=True, random_affine=True)
    mask = make_update_mask(B, H, T, 16, 0.5, seed=441)
    skip = np.repeat(mask == 0, 16, axis=2)[:, :, :T]
    t = dev(x)
    o1, W1 = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                         t["gamma"], t["beta"], dual=True, chunk=16,
                         update_mask=torch.from_numpy(mask).cuda())
    x.eta_logit[skip] = -np.inf
    t = dev(x)
    o2, W2, _ = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                   t["W0"], t["gamma"], t["beta"], dual=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(W1, W2)
    dout, dWf = make_cotangents(B, H, T, 64, seed=442)
    g = gpu_bwd(x, dout, dWf, dual=True)
    assert np.all(g["deta_logit"][skip] == 0.0)
    compare(g, ref_bwd(x, dout, dWf, dual=True), TOL[True])


def test_dual_silu_backward():
    say("case dual backward silu_qk")
    x = make_case(2, 2, 50, 64, seed=450, dual=True, chunk=16, in_bf16=True, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 50, 64, seed=451)
    compare(gpu_bwd(x, dout, dWf, dual=True, silu_qk=True),
            ref_bwd(x, dout, dWf, dual=True, silu_qk=True), TOL[True])


def test_dual_autograd_function_matches_backward():
    say("case dual autograd")
    x = make_case(2, 2, 33, 64, seed=460, dual=True, chunk=16, random_affine=True)
    dout, dWf = make_cotangents(2, 2, 33, 64, seed=461)
    t = dev(x)
    leaves = {k: v.clone().requires_grad_() for k, v in t.items()}
    out, Wf = ttt.ttt_linear(*[leaves[k] for k in ("q", "k", "v", "eta_logit", "gate_logit",
                                                   "W0", "gamma", "beta")], ln="st", dual=True)
    ((out * cot(dout)).sum() + (Wf * cot(dWf)).sum()).backward()
    r = ref_bwd(x, dout, dWf, dual=True)
    names = dict(q="dq", k="dk", v="dv", eta_logit="deta_logit", gate_logit="dgate_logit",
                 W0="dW0", gamma="dgamma", beta="dbeta")
    for leaf, key in names.items():
        assert_close(leaves[leaf].grad.cpu().numpy(), r[key], 1e-4, f"autograd {key}")


def test_full_size_dual_backward_sampled():
    workload, head = "h2048_T8192_dual16_bf16", 11
    say(f"case dual backward full size {workload} head {head}")
    x = make_inputs(workload)
    B, H, T, d = x.q.shape
    dout, dWf = make_cotangents(B, H, T, d, seed=470)
    g = gpu_bwd(x, dout, dWf, dual=True)
    xs, ds, dWs, (bs, hs) = _sampled(x, dout, dWf, head)
    r = ref_bwd(xs, ds, dWs, dual=True)
    per_scan(g, r, bs, hs, ("dq", "dk", "dv", "dgate_logit", "deta_logit", "dW0"), TOL[True])
    assert_close(g["dgamma"][head], r["dgamma"].sum(axis=0), TOL[True], "dgamma")
    assert_close(g["dbeta"][head], r["dbeta"].sum(axis=0), TOL[True], "dbeta")
