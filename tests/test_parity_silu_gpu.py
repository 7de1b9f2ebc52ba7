"""GPU parity of the :mlp variant (TTT_SILU_QK: SiLU on keys and queries
before the inner model) against the float64 oracle with ``silu_qk=True``.

The forward runs on both kernels; the backward on the matrix-core path.  On
the bf16-input matrix-core path the activated q and k are rounded to bf16
(the MFMA operand type), which the bf16 tolerance covers.  Tolerances:
relative max error 1e-4 (fp32 inputs), 2e-2 (bf16 inputs)."""
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


def close(got, want, tol, what):
    err = oracle.rel_max_err(got, want)
    say(f"    {what}: rel max err {err:.3g} (tol {tol:g})")
    assert np.all(np.isfinite(got)) and err <= tol, f"{what}: {err:.3g}"


FWD = [(64, ln, bf16, False, 16) for ln in ("st", "exact", "none") for bf16 in (False, True)]
FWD += [(64, "st", True, True, 16), (64, "exact", False, True, 16), (32, "st", False, False, 1),
        (32, "exact", True, True, 5), (128, "st", True, False, 1)]


@pytest.mark.parametrize("d,ln,bf16,dual,chunk", FWD)
def test_silu_forward_parity(d, ln, bf16, dual, chunk):
    T = 3 * 16 + 7
    say(f"case silu fwd d={d} ln={ln} bf16={bf16} dual={dual} chunk={chunk}")
    x = make_case(2, 3, T, d, seed=500 + d, ln=ln, in_bf16=bf16, dual=dual, chunk=chunk,
                  random_affine=True)
    t = dev(x)
    out, W = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                         t["gamma"], t["beta"], ln=ln, dual=dual, chunk=chunk, silu_qk=True)
    torch.cuda.synchronize()
    ro, rW = oracle.ttt_linear_forward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                       x.beta, ln=ln, dual=dual, chunk=chunk, silu_qk=True)
    close(out.cpu().numpy(), ro, TOL[bf16], "out")
    close(W.cpu().numpy(), rW, TOL[bf16], "W_final")


def test_silu_with_chunk_mask():
    say("case silu + mask")
    x = make_case(2, 2, 70, 64, seed=510, in_bf16=True, dual=True, chunk=16, random_affine=True)
    mask = make_update_mask(2, 2, 70, 16, 0.5, seed=511)
    t = dev(x)
    out, W = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                         t["gamma"], t["beta"], dual=True, chunk=16, silu_qk=True,
                         update_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    ro, rW = oracle.ttt_linear_forward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                       x.beta, dual=True, chunk=16, silu_qk=True,
                                       update_mask=mask)
    close(out.cpu().numpy(), ro, 2e-2, "out")
    close(W.cpu().numpy(), rW, 2e-2, "W_final")


def gpu_bwd(x, dout, dWf):
    t = dev(x)
    gam = None if x.ln == "none" else t["gamma"]
    bet = None if x.ln == "none" else t["beta"]
    _, _, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                   t["W0"], gam, bet, ln=x.ln, silu_qk=True)
    g = ttt.backward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], gam, bet, rec,
                     torch.from_numpy(dout).cuda(), torch.from_numpy(dWf).cuda(), ln=x.ln,
                     silu_qk=True)
    torch.cuda.synchronize()
    return {k: None if v is None else v.cpu().numpy() for k, v in g.items()}


@pytest.mark.parametrize("ln", ["st", "exact", "none"])
@pytest.mark.parametrize("bf16", [False, True])
def test_silu_backward_parity(ln, bf16):
    T = 53
    say(f"case silu bwd ln={ln} bf16={bf16}")
    x = make_case(2, 3, T, 64, seed=520, ln=ln, in_bf16=bf16, random_affine=True)
    dout, dWf = make_cotangents(2, 3, T, 64, seed=521)
    g = gpu_bwd(x, dout, dWf)
    r = oracle.ttt_linear_backward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                   x.beta, dout, dWf, ln=ln, silu_qk=True)
    for key in GRADS:
        if r[key] is None:
            continue
        close(g[key], r[key], TOL[bf16], key)


def test_silu_full_size_sampled():
    # hidden 1024, T = 4096, bf16 inputs: forward and backward, all batches of one head
    say("case silu full size h1024_T4096_bf16")
    x = make_inputs("h1024_T4096_bf16")
    B, H, T, d = x.q.shape
    dout, dWf = make_cotangents(B, H, T, d, seed=530)
    t = dev(x)
    out, W, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                     t["W0"], t["gamma"], t["beta"], silu_qk=True)
    g = ttt.backward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["gamma"],
                     t["beta"], rec, torch.from_numpy(dout).cuda(), torch.from_numpy(dWf).cuda(),
                     silu_qk=True)
    torch.cuda.synchronize()
    head = 9
    pairs = [(b, head) for b in range(B)]
    xs = x.subset(pairs)
    cut = lambda a: np.ascontiguousarray(a[:, head][None])
    ro, rW = oracle.ttt_linear_forward(xs.q, xs.k, xs.v, xs.eta_logit, xs.gate_logit, xs.W0,
                                       xs.gamma, xs.beta, silu_qk=True)
    o_np, W_np = out.cpu().numpy(), W.cpu().numpy()
    for b in range(B):   # every sampled scan on its own
        close(o_np[b, head], ro[0, b], 2e-2, f"out[{b},{head}]")
        close(W_np[b, head], rW[0, b], 2e-2, f"W_final[{b},{head}]")
    r = oracle.ttt_linear_backward(xs.q, xs.k, xs.v, xs.eta_logit, xs.gate_logit, xs.W0,
                                   xs.gamma, xs.beta, cut(dout), cut(dWf), silu_qk=True)
    for key in ("dq", "dk", "dv", "dgate_logit", "deta_logit", "dW0"):
        gk = g[key].cpu().numpy()
        for b in range(B):
            close(gk[b, head], r[key][0, b], 2e-2, f"{key}[{b},{head}]")
    close(g["dgamma"][head].cpu().numpy(), r["dgamma"].sum(0), 2e-2, "dgamma")
    close(g["dbeta"][head].cpu().numpy(), r["dbeta"].sum(0), 2e-2, "dbeta")
