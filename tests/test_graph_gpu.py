"""HIP graph capture of the C-ABI entry points.

Every entry point only launches kernels on the caller's stream: it allocates
nothing, clears nothing with a memset and never waits on the host, so a
caller can capture it in a HIP graph (here through ``torch.cuda.graph``) and
replay it without launch overhead.  Each case captures one call (or a
recording forward plus its backward) on static input tensors, then three
times copies new seeded values into those inputs, runs the same call eagerly
into fresh outputs, replays the graph, and requires the graph's outputs to
equal the eager ones bit for bit (the kernels are deterministic: no atomics,
fixed summation orders).  The eager work and the synchronisations between
replays are deliberate: a graph must not depend on what ran before it.
"""
import sys

import numpy as np
import pytest

from test_rnn_layer_ttt_amd.inputs import (make_case, make_cotangents, make_mlp_case,
                                           make_projection_case)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, dt=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(dt) if dt is not None else t


def scan_tensors(x, bf16):
    dt = torch.bfloat16 if bf16 else torch.float32
    return dict(q=to_dev(x.q, dt), k=to_dev(x.k, dt), v=to_dev(x.v, dt),
                eta_logit=to_dev(x.eta_logit, dt), gate_logit=to_dev(x.gate_logit, dt),
                W0=to_dev(x.W0), gamma=to_dev(x.gamma), beta=to_dev(x.beta))


def replay_check(static, fresh, call, label):
    """Capture ``call(static)``; for each dict of new input tensors in
    ``fresh``, copy it into ``static``, run ``call`` eagerly, replay, compare."""
    torch.cuda.synchronize()
    call(static)                     # loads the kernels before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = call(static)
    torch.cuda.synchronize()
    for r, new in enumerate(fresh):
        for key, t in new.items():
            static[key].copy_(t)
        torch.cuda.synchronize()
        ref = [o.clone() for o in call(static)]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"{label}: replay {r}, output {i} differs from eager"
        say(f"  {label}: replay {r} equals the eager call")


@pytest.mark.parametrize("d,ln,bf16,dual", [
    (64, "st", True, False),      # matrix-core per-token scan
    (64, "exact", False, False),
    (64, "st", True, True),       # matrix-core dual form
    (32, "st", False, False),     # vector-ALU scan
])
def test_forward_in_a_graph(d, ln, bf16, dual):
    say(f"case graph forward d={d} ln={ln} bf16={bf16} dual={dual}")
    mk = lambda seed: scan_tensors(make_case(2, 2, 83, d, seed=seed, ln=ln, dual=dual, chunk=16,
                                             in_bf16=bf16, random_affine=True), bf16)
    call = lambda s: ttt.forward(s["q"], s["k"], s["v"], s["eta_logit"], s["gate_logit"],
                                 s["W0"], s["gamma"], s["beta"], ln=ln, dual=dual, chunk=16)
    replay_check(mk(700), [mk(701 + r) for r in range(3)], call, "forward")


@pytest.mark.parametrize("ln,bf16", [("exact", False), ("st", True)])
def test_forward_record_and_backward_in_a_graph(ln, bf16):
    say(f"case graph forward_record + backward ln={ln} bf16={bf16}")
    B, H, T, d = 2, 2, 53, 64

    def mk(seed):
        s = scan_tensors(make_case(B, H, T, d, seed=seed, ln=ln, in_bf16=bf16,
                                   random_affine=True), bf16)
        dout, dWf = make_cotangents(B, H, T, d, seed=seed + 50)
        s["dout"], s["dWf"] = to_dev(dout), to_dev(dWf)
        return s

    def call(s):
        args = [s[n] for n in ("q", "k", "v", "eta_logit", "gate_logit")]
        out, Wf, rec = ttt.forward_record(*args, s["W0"], s["gamma"], s["beta"], ln=ln)
        gr = ttt.backward(*args, s["gamma"], s["beta"], rec, s["dout"], s["dWf"], ln=ln)
        return [out, Wf] + [gr[n] for n in sorted(gr) if gr[n] is not None]

    replay_check(mk(710), [mk(711 + r) for r in range(3)], call, "record+backward")


def test_two_layer_forward_in_a_graph():
    say("case graph two-layer forward (dual form, bf16)")

    def mk(seed):
        x, W1 = make_mlp_case(2, 2, 67, 64, seed=seed, dual=True, chunk=16, in_bf16=True,
                              random_affine=True)
        s = scan_tensors(x, True)
        s["W1"] = to_dev(W1)
        return s

    call = lambda s: ttt.mlp_forward(s["q"], s["k"], s["v"], s["eta_logit"], s["gate_logit"],
                                     s["W1"], s["W0"], s["gamma"], s["beta"], dual=True,
                                     chunk=16)
    replay_check(mk(720), [mk(721 + r) for r in range(3)], call, "two-layer forward")


def test_projections_in_a_graph():
    say("case graph input projections")

    def mk(seed):
        x, w, b = make_projection_case(2, 300, 256, 4, 64, seed=seed, with_bias=True)
        return dict(x=to_dev(x, torch.bfloat16), w=to_dev(w, torch.bfloat16), b=to_dev(b))

    call = lambda s: ttt.project(s["x"], s["w"], s["b"])
    replay_check(mk(730), [mk(731 + r) for r in range(3)], call, "projections")
