"""GPU parity of the inner LayerNorm where its statistic is hard to get right.

"Edifice.Recurrent.TTT" ("Paper-Faithful Implementation", item 3) puts the
LayerNorm there because prediction magnitudes drift.  Two regimes test the
kernels' mean/variance of z = W k against the float64 oracle:

* off-centre: the feature mean of z is hundreds to a thousand times its
  spread (W0 with a large common row component, or targets v with a large
  constant mean, which the straight-through update turns into a common row of
  W).  A one-pass E[z^2] - E[z]^2 in fp32 loses the variance here;
* degenerate (the reading that a zero variance gives xhat = 0): W0 = 0, so
  z_0 = 0 exactly and the first prediction is beta.

Every case compares out and W_final (relative max error per tensor, 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs) and, where a recording forward exists, every
recorded inner-gradient vector delta_t, the quantity the statistic feeds
directly.  The oracle's own LayerNorm statistics are printed and checked to be
in the intended regime.
"""
import sys

import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import make_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402

TOL = {False: 1e-4, True: 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x):
    dt = torch.bfloat16 if x.in_bf16 else torch.float32
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(q=f(x.q), k=f(x.k), v=f(x.v), eta_logit=f(x.eta_logit),
                gate_logit=f(x.gate_logit), W0=g(x.W0), gamma=g(x.gamma), beta=g(x.beta))


def check(got, ref, tol, what):
    err = oracle.rel_max_err(got, ref)
    say(f"    {what}: rel max err {err:.3g} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: rel max err {err:.3g} > {tol:g}"
    return err


def run_case(x, ln, dual, force_valu=False, record=False):
    """GPU forward (and the recorded deltas when ``record``) against the oracle."""
    t = dev(x)
    args = (t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"], t["gamma"],
            t["beta"])
    if record:
        out, W, rec = ttt.forward_record(*args, ln=ln, dual=dual)
    else:
        out, W = ttt.forward(*args, ln=ln, dual=dual, chunk=16, force_valu=force_valu)
    torch.cuda.synchronize()
    ro, rW, st = oracle.ttt_linear_forward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0,
                                           x.gamma, x.beta, ln=ln, dual=dual, chunk=16,
                                           return_ln_stats=True)
    tol = TOL[x.in_bf16]
    check(out.cpu().numpy(), ro, tol, "out")
    check(W.cpu().numpy(), rW, tol, "W_final")
    if record:
        # the record starts with delta_t, [B,H,T,d] fp32
        B, H, T, d = x.q.shape
        delta = rec[:B * H * T * d * 4].view(torch.float32).reshape(B, H, T, d)
        check(delta.cpu().numpy(), st["delta"], tol, "delta")
    return st


def off_centre(stats):
    r = np.abs(stats["mean"]) / np.maximum(stats["std"], 1e-30)
    say(f"    |mean(z)|/std(z): median {np.median(r):.3g}, max {r.max():.3g}")
    return r


# ---------------------------------------------------------------------------
# off-centre LayerNorm inputs, long sequences
# ---------------------------------------------------------------------------
OFF = [  # (name, generator options, ln, the least max |mean|/std the case must reach)
    ("v+10", dict(v_mean=10.0), "st", 200.0),
    ("W0 common row 100", dict(w0_common_row=100.0), "st", 1000.0),
    ("W0 common row 100", dict(w0_common_row=100.0), "exact", 500.0),
    ("v+10, W0 common row 100", dict(v_mean=10.0, w0_common_row=100.0), "st", 1000.0),
]


@pytest.mark.parametrize("name,opts,ln,reach", OFF, ids=[f"{o[0]}-{o[2]}" for o in OFF])
def test_off_centre_per_token_fp32(name, opts, ln, reach):
    say(f"case off-centre {name} ln={ln} per-token fp32 T=4096")
    x = make_case(1, 2, 4096, 64, seed=500, ln=ln, random_affine=True, **opts)
    st = run_case(x, ln, dual=False, record=True)
    assert off_centre(st).max() >= reach


@pytest.mark.parametrize("ln", ["st", "exact"])
def test_off_centre_vector_alu_kernel(ln):
    say(f"case off-centre W0 common row 100 ln={ln} vector-ALU kernel, d=64, T=4096")
    x = make_case(1, 2, 4096, 64, seed=501, ln=ln, random_affine=True, w0_common_row=100.0)
    st = run_case(x, ln, dual=False, force_valu=True)
    assert off_centre(st).max() >= 500.0


@pytest.mark.parametrize("d", [32, 128])
def test_off_centre_other_head_sizes(d):
    say(f"case off-centre W0 common row 100 d={d} T=2048")
    x = make_case(1, 2, 2048, d, seed=502, ln="st", random_affine=True, w0_common_row=100.0)
    st = run_case(x, "st", dual=False)
    assert off_centre(st).max() >= 200.0


@pytest.mark.parametrize("ln", ["st", "exact"])
def test_off_centre_dual_form(ln):
    say(f"case off-centre W0 common row 100 ln={ln} dual chunk 16, fp32, T=4096")
    x = make_case(1, 2, 4096, 64, seed=503, ln=ln, random_affine=True, w0_common_row=100.0)
    st = run_case(x, ln, dual=True, record=True)
    assert off_centre(st).max() >= 500.0


@pytest.mark.parametrize("dual", [False, True])
def test_off_centre_bf16_inputs(dual):
    say(f"case off-centre v+10, W0 common row 100, bf16 inputs, dual={dual}, T=4096")
    x = make_case(1, 2, 4096, 64, seed=504, in_bf16=True, v_mean=10.0, w0_common_row=100.0)
    st = run_case(x, "st", dual=dual)
    assert off_centre(st).max() >= 500.0


# ---------------------------------------------------------------------------
# degenerate LayerNorm: W0 = 0, so z_0 = 0 (zero variance) and pred_0 = beta
# ---------------------------------------------------------------------------
DEG = []
for ln in ("st", "exact"):
    for bf16 in (False, True):
        DEG.append((64, ln, bf16, False, False))      # matrix-core, per-token
        DEG.append((64, ln, bf16, True, False))       # matrix-core, dual form
        DEG.append((64, ln, bf16, False, True))       # vector-ALU, per-token
    DEG.append((32, ln, False, False, False))
    DEG.append((128, ln, False, True, False))


@pytest.mark.parametrize("d,ln,bf16,dual,valu", DEG)
def test_zero_initial_weight(d, ln, bf16, dual, valu):
    say(f"case W0 = 0 d={d} ln={ln} bf16={bf16} dual={dual} valu={valu}")
    x = make_case(2, 3, 100, d, seed=510 + d, ln=ln, in_bf16=bf16, random_affine=True)
    x.W0[:] = 0.0
    st = run_case(x, ln, dual, force_valu=valu, record=(d == 64 and not valu))
    assert np.all(st["std"][..., 0] == 0.0)        # the first token's z is exactly 0
