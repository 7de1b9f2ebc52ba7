"""GPU parity of the input projections (``ttt_linear_project``, through the
C ABI) against the float64 oracle (``oracle.input_projections``) on the same
bf16 x and weights.

fp32 outputs: relative max error (per tensor) <= 1e-4, the fp32 tolerance.
The products of bf16 values are exact in fp32, so the only difference is the
fp32 summation order.  bf16 outputs: every element within one bf16 rounding
step of the float64 value (|got - ref| <= 2^-8 |ref|, plus 1e-6 of the
tensor's largest value for results that cancel to near zero): the kernel
rounds its fp32 sum once, so a value can differ from the rounded float64
value only where the two sit on either side of a rounding boundary."""
import sys

import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import make_case, make_projection_case, round_to_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402

NAMES = ("q", "k", "v", "eta_logit", "gate_logit")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_project(x, w, b, out_bf16):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xt = dev(x).to(torch.bfloat16)
    wt = dev(w).to(torch.bfloat16)
    bt = None if b is None else dev(b)
    outs = ttt.project(xt, wt, bt, out_bf16=out_bf16)
    torch.cuda.synchronize()
    return [o.float().cpu().numpy() for o in outs]


def compare(got, ref, out_bf16, what=""):
    for name, g, r in zip(NAMES, got, ref):
        assert g.shape == r.shape, (name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), name
        if out_bf16:
            bound = 2.0 ** -8 * np.abs(r) + 1e-6 * np.max(np.abs(r))
            worst = float(np.max(np.abs(g - r) - bound)) if r.size else -1.0
            say(f"    {what}{name}: worst excess over one rounding step {worst:.3g}")
            assert worst <= 0.0, name
        else:
            err = oracle.rel_max_err(g, r)
            say(f"    {what}{name}: rel max err {err:.3g}")
            assert err <= 1e-4, (name, err)


@pytest.mark.parametrize("hidden", [32, 96, 256])
@pytest.mark.parametrize("H", [1, 3])
@pytest.mark.parametrize("out_bf16", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_small_projection_parity(hidden, H, out_bf16, with_bias):
    B, T = 2, 37
    say(f"case project hidden={hidden} H={H} bf16={out_bf16} bias={with_bias}")
    x, w, b = make_projection_case(B, T, hidden, H, 64, seed=500 + hidden + H, with_bias=with_bias)
    compare(gpu_project(x, w, b, out_bf16), oracle.input_projections(x, w, b), out_bf16)


@pytest.mark.parametrize("out_bf16", [False, True])
@pytest.mark.parametrize("B,T,H", [(3, 200, 2), (1, 129, 260), (2, 1, 5), (2, 300, 8),
                                   (5, 70, 3)])
def test_ragged_tiles_and_many_heads(B, T, H, out_bf16):
    # token tiles (256 tokens) across batch boundaries and a ragged last tile
    # (with bf16 results also sequence boundaries inside a wave's 64 staged
    # rows, for T below and above 64); more than 256 heads puts the eta rows
    # in two tiles, the second one mostly empty
    say(f"case project B={B} T={T} H={H} bf16={out_bf16}")
    x, w, b = make_projection_case(B, T, 64, H, 64, seed=510 + T, with_bias=True)
    compare(gpu_project(x, w, b, out_bf16), oracle.input_projections(x, w, b), out_bf16)


@pytest.mark.parametrize("hidden", [64, 128, 160, 192])
def test_step_counts_around_the_ring(hidden):
    # 2, 4, 5 and 6 K steps of 32: no steady-state step, and one pair of them
    # followed by three or four closing steps
    B, T, H = 1, 300, 2
    say(f"case project hidden={hidden} (K steps {hidden // 32})")
    x, w, b = make_projection_case(B, T, hidden, H, 64, seed=550 + hidden, with_bias=True)
    compare(gpu_project(x, w, b, True), oracle.input_projections(x, w, b), True)


def test_one_hot_rows_route_every_output():
    # each weight row selects one coordinate of x: every output element is an
    # exact copy of an x value, so bf16 outputs must match bit for bit
    B, T, H, d = 2, 50, 2, 64
    R = 4 * d + 1
    hidden = 32 * ((H * R + 31) // 32)
    rng = np.random.default_rng(7)
    x = round_to_bf16(rng.standard_normal((B, T, hidden)).astype(np.float32))
    sel = rng.permutation(hidden)[:H * R].reshape(H, R)
    w = np.zeros((H, R, hidden), np.float32)
    for h in range(H):
        w[h, np.arange(R), sel[h]] = 1.0
    got = gpu_project(x, w, None, True)
    ref = oracle.input_projections(x, w)
    for name, g, r in zip(NAMES, got, ref):
        assert np.array_equal(g, r), name


def test_repeatable_bits():
    x, w, b = make_projection_case(2, 300, 256, 4, 64, seed=520, with_bias=True)
    a = gpu_project(x, w, b, True)
    c = gpu_project(x, w, b, True)
    for u, v in zip(a, c):
        assert np.array_equal(u, v)


def test_projection_then_scan_matches_the_oracle_chain():
    # the projections feed the scan directly: the bf16 results of the GPU
    # projection go through the GPU scan; the oracle runs its projection,
    # rounds to bf16 (the scan's input type) and runs its scan
    B, T, hidden, H, d = 2, 90, 128, 3, 64
    say("case project -> scan")
    x, w, b = make_projection_case(B, T, hidden, H, d, seed=530, with_bias=True)
    s = make_case(B, H, T, d, seed=531, random_affine=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v, eta, gate = ttt.project(dev(x).to(torch.bfloat16), dev(w).to(torch.bfloat16), dev(b))
    out, Wf = ttt.forward(q, k, v, eta, gate, dev(s.W0), dev(s.gamma), dev(s.beta), ln="st")
    torch.cuda.synchronize()
    rq, rk, rv, reta, rgate = (round_to_bf16(a.astype(np.float32))
                               for a in oracle.input_projections(x, w, b))
    ro, rW = oracle.ttt_linear_forward(rq, rk, rv, reta, rgate, s.W0, s.gamma, s.beta, ln="st")
    e_o = oracle.rel_max_err(out.cpu().numpy(), ro)
    e_w = oracle.rel_max_err(Wf.cpu().numpy(), rW)
    say(f"    out {e_o:.3g}, W_final {e_w:.3g}")
    assert e_o <= 2e-2 and e_w <= 2e-2


@pytest.mark.parametrize("B,T,hidden,H", [(16, 4096, 1024, 16), (8, 8192, 2048, 32)])
def test_full_size_sampled_tokens(B, T, hidden, H):
    # the hidden-1024 and hidden-2048 workloads' shapes, as the benchmark
    # launches them; the oracle checks 64 sampled tokens of every head
    d = 64
    say(f"case project full size B={B} T={T} hidden={hidden} H={H}")
    x, w, _ = make_projection_case(B, T, hidden, H, d, seed=540 + H)
    got = gpu_project(x, w, None, True)
    rng = np.random.default_rng(541)
    bs = rng.integers(0, B, 64)
    ts = rng.integers(0, T, 64)
    ref = oracle.input_projections(x[bs, ts][None], w)     # [1, H, 64, ...]
    for name, g, r in zip(NAMES, got, ref):
        gs = np.stack([g[bb, :, tt] for bb, tt in zip(bs, ts)], axis=1)[None]
        bound = 2.0 ** -8 * np.abs(r) + 1e-6 * np.max(np.abs(r))
        assert np.all(np.abs(gs - r) <= bound), name
