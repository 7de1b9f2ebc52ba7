"""GPU parity: the HIP scan (through the C ABI) against the float64 oracle.

Small cases are compared element by element over every output; the five
named full-size workloads run on the GPU exactly as the benchmark launches
them and are compared on sampled (batch, head) scans, which the oracle
computes at full sequence length.  Tolerances: relative max error
(max|gpu - ref| / max|ref|, per tensor) 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs, the oracle being fed the same bf16-rounded values.
"""
import sys

import numpy as np
import pytest

import oracle
from test_rnn_layer_ttt_amd.inputs import make_case, make_inputs

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


def gpu_run(x, ln=None, dual=None, chunk=None, **kw):
    t = dev(x)
    out, W = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                         t["gamma"], t["beta"], ln=x.ln if ln is None else ln,
                         dual=x.dual if dual is None else dual,
                         chunk=x.chunk if chunk is None else chunk, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), W.cpu().numpy()


def ref_run(x, ln=None, dual=None, chunk=None):
    return oracle.ttt_linear_forward(x.q, x.k, x.v, x.eta_logit, x.gate_logit, x.W0, x.gamma,
                                     x.beta, ln=x.ln if ln is None else ln,
                                     dual=x.dual if dual is None else dual,
                                     chunk=x.chunk if chunk is None else chunk)


def assert_close(got, ref, tol, what):
    err = oracle.rel_max_err(got, ref)
    say(f"    {what}: rel max err {err:.3g} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: rel max err {err:.3g} > {tol:g}"


# ---------------------------------------------------------------------------
# small cases: every output element, several LDS tiles plus a ragged tail
# ---------------------------------------------------------------------------
CASES = []
for d in (16, 32, 64, 128):
    tile = 2048 // d
    for ln in ("st", "exact", "none"):
        for bf16 in (False, True):
            for dual, chunk in ((False, 1), (True, 16), (True, 5)):
                CASES.append((d, ln, bf16, dual, chunk, 2 * tile + 13))


@pytest.mark.parametrize("d,ln,bf16,dual,chunk,T", CASES)
def test_small_parity(d, ln, bf16, dual, chunk, T):
    say(f"case d={d} ln={ln} bf16={bf16} dual={dual} chunk={chunk} T={T}")
    x = make_case(2, 3, T, d, seed=100 + d + T, ln=ln, dual=dual, chunk=chunk, in_bf16=bf16,
                  random_affine=True)
    out, W = gpu_run(x)
    ro, rW = ref_run(x)
    assert_close(out, ro, TOL[bf16], "out")
    assert_close(W, rW, TOL[bf16], "W_final")


VALU64 = [(ln, bf16, dual, chunk) for ln in ("st", "exact", "none") for bf16 in (False, True)
          for dual, chunk in ((False, 1), (True, 16), (True, 5))]


@pytest.mark.parametrize("ln,bf16,dual,chunk", VALU64)
def test_small_parity_vector_alu_d64(ln, bf16, dual, chunk):
    # the vector-ALU kernel at d = 64, where a plain call runs the matrix-core one
    say(f"case vector-ALU d=64 ln={ln} bf16={bf16} dual={dual} chunk={chunk}")
    assert ttt.ttt_linear_kernel(64, ttt.mode_bits(ln, dual, bf16, force_valu=True),
                                 chunk) == "scan_valu"
    x = make_case(2, 3, 77, 64, seed=150, ln=ln, dual=dual, chunk=chunk, in_bf16=bf16,
                  random_affine=True)
    out, W = gpu_run(x, force_valu=True)
    ro, rW = ref_run(x)
    assert_close(out, ro, TOL[bf16], "out")
    assert_close(W, rW, TOL[bf16], "W_final")


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 64, 65])
@pytest.mark.parametrize("ln,dual", [("st", False), ("exact", False), ("st", True)])
def test_short_and_ragged_sequences(T, ln, dual):
    say(f"case T={T} ln={ln} dual={dual}")
    x = make_case(3, 2, T, 64, seed=T, ln=ln, dual=dual, chunk=16, random_affine=True)
    out, W = gpu_run(x)
    ro, rW = ref_run(x)
    assert_close(out, ro, 1e-4, "out")
    assert_close(W, rW, 1e-4, "W_final")


# ---------------------------------------------------------------------------
# closed forms and invariants on the GPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ln,dual", [("st", False), ("exact", False), ("none", False),
                                     ("st", True)])
def test_eta_zero_leaves_state_and_gates_W0_q(ln, dual):
    say(f"case eta=-inf ln={ln} dual={dual}")
    x = make_case(2, 2, 70, 64, seed=7, random_affine=True)
    x.eta_logit[:] = -np.inf
    out, W = gpu_run(x, ln=ln, dual=dual, chunk=16)
    assert np.array_equal(W, x.W0)
    want = np.einsum("bhij,bhtj->bhti", x.W0.astype(np.float64), x.q.astype(np.float64))
    want = want / (1.0 + np.exp(-x.gate_logit.astype(np.float64)))
    assert_close(out, want, 1e-5, "out")


def test_gate_limits():
    say("case gate limits")
    x = make_case(2, 2, 50, 64, seed=8, random_affine=True)
    x.gate_logit[:] = -np.inf
    out_shut, W1 = gpu_run(x)
    assert np.all(out_shut == 0.0)
    x.gate_logit[:] = np.inf
    out_open, W2 = gpu_run(x)
    assert np.array_equal(W1, W2)
    ro, _ = ref_run(x)
    assert_close(out_open, ro, 1e-4, "out (gate open)")


def test_overwrite_identity():
    """No LN, ||k||^2 = 2d and eta = 1/(2d): each step writes v_t at k_t."""
    say("case overwrite identity")
    d = 64
    x = make_case(2, 2, 40, d, seed=9)
    k = x.k.astype(np.float64)
    x.k = (k / np.linalg.norm(k, axis=-1, keepdims=True) * np.sqrt(2.0 * d)).astype(np.float32)
    x.q = x.k.copy()
    x.eta_logit[:] = 0.0
    out, _ = gpu_run(x, ln="none")
    want = x.v.astype(np.float64) / (1.0 + np.exp(-x.gate_logit.astype(np.float64)))
    assert_close(out, want, 1e-4, "out")


def test_empty_sequence_copies_state():
    say("case T=0")
    x = make_case(2, 3, 0, 64, seed=10, random_affine=True)
    out, W = gpu_run(x)
    assert out.shape == (2, 3, 0, 64)
    assert np.array_equal(W, x.W0)


def test_state_in_place_and_not_written():
    say("case in-place state")
    x = make_case(2, 2, 45, 64, seed=11, random_affine=True)
    t = dev(x)
    W0 = t["W0"].clone()
    out, Wf = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], W0,
                          t["gamma"], t["beta"], W_final=W0)
    torch.cuda.synchronize()
    assert Wf.data_ptr() == W0.data_ptr()
    ro, rW = ref_run(x)
    assert_close(out.cpu().numpy(), ro, 1e-4, "out")
    assert_close(W0.cpu().numpy(), rW, 1e-4, "W_final (in place)")
    # W_final = NULL: nothing written, out unchanged
    status = ttt.ttt_linear_forward(
        t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["eta_logit"].data_ptr(),
        t["gate_logit"].data_ptr(), t["W0"].data_ptr(), t["gamma"].data_ptr(),
        t["beta"].data_ptr(), out.data_ptr(), None, 2, 2, 45, 64, 0, 1,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert status == ttt.TTT_OK
    assert_close(out.cpu().numpy(), ro, 1e-4, "out (no W_final)")


@pytest.mark.parametrize("d,ln,dual,chunk", [(64, "st", False, 1), (64, "exact", False, 1),
                                             (64, "st", True, 16), (32, "st", False, 1),
                                             (32, "exact", True, 5)])
def test_resume_equals_one_call(d, ln, dual, chunk):
    """Two calls chained through W_final equal one call over the whole sequence.

    The vector-ALU scan takes every token the same way in both, so the match
    is bitwise.  The matrix-core scan forms z of the first tile of a call from
    W directly and of later tiles through the one-tile-ahead correction: the
    same value in exact arithmetic, rounded differently, so it must match to
    the fp32 tolerance.
    """
    say(f"case resume d={d} ln={ln} dual={dual}")
    T1, T = 80, 150
    x = make_case(2, 2, T, d, seed=12, ln=ln, dual=dual, chunk=chunk, random_affine=True,
                  in_bf16=True)
    t = dev(x)
    full_o, full_W = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                 t["W0"], t["gamma"], t["beta"], ln=ln, dual=dual, chunk=chunk)
    cut = lambda a, sl: a[:, :, sl].contiguous()
    first = [cut(t[n], slice(0, T1)) for n in ("q", "k", "v", "eta_logit", "gate_logit")]
    second = [cut(t[n], slice(T1, T)) for n in ("q", "k", "v", "eta_logit", "gate_logit")]
    o1, W1 = ttt.forward(*first, t["W0"], t["gamma"], t["beta"], ln=ln, dual=dual, chunk=chunk)
    o2, W2 = ttt.forward(*second, W1, t["gamma"], t["beta"], ln=ln, dual=dual, chunk=chunk)
    torch.cuda.synchronize()
    o12 = torch.cat([o1, o2], dim=2)
    kernel = ttt.ttt_linear_kernel(d, ttt.mode_bits(ln, dual, True), chunk)
    if kernel == "scan_valu":
        assert torch.equal(o12, full_o)
        assert torch.equal(W2, full_W)
    else:
        assert_close(o12.cpu().numpy(), full_o.cpu().numpy(), 1e-5, "out (resumed vs one call)")
        assert_close(W2.cpu().numpy(), full_W.cpu().numpy(), 1e-5, "W_final (resumed vs one call)")
    ro, rW = ref_run(x)
    assert_close(o12.cpu().numpy(), ro, 2e-2, "out vs oracle")


def test_deterministic_and_batch_split_invariant():
    say("case determinism / batch split")
    x = make_case(3, 4, 100, 64, seed=13, random_affine=True)
    o1, W1 = gpu_run(x)
    o2, W2 = gpu_run(x)
    assert np.array_equal(o1, o2) and np.array_equal(W1, W2)
    pairs = [(2, 3), (0, 1), (1, 1)]
    s = x.subset(pairs)
    o3, W3 = gpu_run(s)
    for n, (b, h) in enumerate(pairs):
        assert np.array_equal(o3[0, n], o1[b, h])
        assert np.array_equal(W3[0, n], W1[b, h])


def test_side_stream():
    say("case side stream")
    x = make_case(2, 2, 80, 64, seed=14, random_affine=True)
    t = dev(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, W = ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                             t["gamma"], t["beta"], stream=s)
    s.synchronize()
    ro, rW = ref_run(x)
    assert_close(out.cpu().numpy(), ro, 1e-4, "out")
    assert_close(W.cpu().numpy(), rW, 1e-4, "W_final")


def test_binding_rejects_bad_arguments():
    say("case argument errors")
    x = make_case(1, 2, 16, 64, seed=15)
    t = dev(x)
    with pytest.raises(ValueError):   # out aliases k
        ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                    t["gamma"], t["beta"], out=t["k"])
    with pytest.raises(ValueError):   # d = 48 unsupported
        z = torch.zeros(1, 1, 4, 48, device="cuda")
        ttt.forward(z, z.clone(), z.clone(), torch.zeros(1, 1, 4, device="cuda"), z.clone(),
                    torch.zeros(1, 1, 48, 48, device="cuda"),
                    torch.ones(1, 48, device="cuda"), torch.zeros(1, 48, device="cuda"))
    with pytest.raises(ValueError):   # dual with chunk 0
        ttt.forward(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"], t["W0"],
                    t["gamma"], t["beta"], dual=True, chunk=0)


# ---------------------------------------------------------------------------
# more scans than compute units (several workgroups per CU), and a long sequence
# (thousands of tiles, a ragged last one)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bf16,ln,dual", [(True, "st", False), (False, "exact", False),
                                          (True, "st", True), (False, "none", True)])
def test_more_scans_than_compute_units(bf16, ln, dual):
    say(f"case 600 scans bf16={bf16} ln={ln} dual={dual}")
    x = make_case(B=20, H=30, T=37, d=64, seed=11, ln=ln, dual=dual, chunk=16, in_bf16=bf16,
                  random_affine=True)
    out, W = gpu_run(x)
    pairs = [(0, 0), (19, 29), (7, 13), (13, 2)]
    ro, rW = ref_run(x.subset(pairs))
    for n, (b, h) in enumerate(pairs):
        assert_close(out[b, h], ro[0, n], TOL[bf16], f"out[{b},{h}]")
        assert_close(W[b, h], rW[0, n], TOL[bf16], f"W_final[{b},{h}]")


@pytest.mark.parametrize("bf16,ln", [(True, "st"), (False, "exact")])
def test_long_sequence(bf16, ln):
    say(f"case T=20011 bf16={bf16} ln={ln}")
    x = make_case(B=1, H=2, T=20011, d=64, seed=12, ln=ln, in_bf16=bf16, random_affine=True)
    out, W = gpu_run(x)
    ro, rW = ref_run(x)
    assert_close(out, ro, TOL[bf16], "out")
    assert_close(W, rW, TOL[bf16], "W_final")


# ---------------------------------------------------------------------------
# the named full-size workloads, launched as the benchmark launches them
# ---------------------------------------------------------------------------
SAMPLES = {"tiny_d16_fp32": None}


@pytest.mark.parametrize("name", ["tiny_d16_fp32", "h256_T2048_fp32", "h1024_T4096_bf16",
                                  "h2048_T8192_dual16_bf16", "h2048_T16384_exact_fp32"])
def test_named_workload(name):
    say(f"case workload {name}")
    x = make_inputs(name)
    B, H, T, d = x.q.shape
    out, W = gpu_run(x)
    if name == "tiny_d16_fp32":
        pairs = [(b, h) for b in range(B) for h in range(H)]
    else:
        pairs = [(0, 0), (B - 1, H - 1), (B // 2, (H * 3) // 5)]
    s = x.subset(pairs)
    ro, rW = ref_run(s)
    for n, (b, h) in enumerate(pairs):
        assert_close(out[b, h], ro[0, n], TOL[x.in_bf16], f"out[{b},{h}]")
        assert_close(W[b, h], rW[0, n], TOL[x.in_bf16], f"W_final[{b},{h}]")


@pytest.mark.parametrize("name", ["h256_T2048_fp32", "h1024_T4096_bf16"])
def test_named_workload_vector_alu(name):
    # the per-token workloads on the vector-ALU kernel, as the benchmark times it beside
    say(f"case workload {name} on the vector-ALU kernel")
    x = make_inputs(name)
    B, H, T, d = x.q.shape
    out, W = gpu_run(x, force_valu=True)
    pairs = [(0, 0), (B - 1, H - 1)]
    ro, rW = ref_run(x.subset(pairs))
    for n, (b, h) in enumerate(pairs):
        assert_close(out[b, h], ro[0, n], TOL[x.in_bf16], f"out[{b},{h}]")
        assert_close(W[b, h], rW[0, n], TOL[x.in_bf16], f"W_final[{b},{h}]")
