"""The backward entry point that allocates nothing (ttt_linear_backward_noalloc),
through the C ABI, against ttt_linear_backward with a caller workspace: two
calls in a row on one GPU, the second with a smaller input, each bit for bit
equal to the workspace entry point's result (the same kernels run in the same
order, only the scratch lives elsewhere)."""
import sys

import numpy as np
import pytest

from test_rnn_layer_ttt_amd.inputs import make_case, make_cotangents

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import test_rnn_layer_ttt_amd as ttt  # noqa: E402

GRADS = ("dq", "dk", "dv", "deta_logit", "dgate_logit", "dW0", "dgamma", "dbeta")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(B, H, T, ln, bf16, seed, d=64, chunk=None):
    x = make_case(B, H, T, d, seed=seed, ln=ln, in_bf16=bf16, random_affine=True)
    dout, dWf = make_cotangents(B, H, T, d, seed=seed + 1)
    dt = torch.bfloat16 if bf16 else torch.float32
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    t = dict(q=f(x.q), k=f(x.k), v=f(x.v), eta_logit=f(x.eta_logit), gate_logit=f(x.gate_logit),
             W0=g(x.W0), gamma=g(x.gamma), beta=g(x.beta), dout=g(dout), dWf=g(dWf))
    gam = None if ln == "none" else t["gamma"]
    bet = None if ln == "none" else t["beta"]
    _, _, rec = ttt.forward_record(t["q"], t["k"], t["v"], t["eta_logit"], t["gate_logit"],
                                   t["W0"], gam, bet, ln=ln, dual=chunk is not None,
                                   chunk=chunk or 16)
    return x, t, rec


def outputs(B, H, T, ln, d=64):
    f32 = dict(dtype=torch.float32, device="cuda")
    o = {n: torch.full((B, H, T, d), float("nan"), **f32) for n in ("dq", "dk", "dv",
                                                                    "dgate_logit")}
    o["deta_logit"] = torch.full((B, H, T), float("nan"), **f32)
    o["dW0"] = torch.full((B, H, d, d), float("nan"), **f32)
    o["dgamma"] = None if ln == "none" else torch.full((H, d), float("nan"), **f32)
    o["dbeta"] = None if ln == "none" else torch.full((H, d), float("nan"), **f32)
    return o


def call(noalloc, t, rec, o, B, H, T, ln, bf16, ws=None, d=64, chunk=None):
    p = lambda a: None if a is None else a.data_ptr()
    no_ln = ln == "none"
    mode = ttt.mode_bits(ln, chunk is not None, bf16)
    common = (p(t["q"]), p(t["k"]), p(t["v"]), p(t["eta_logit"]), p(t["gate_logit"]),
              None if no_ln else p(t["gamma"]), None if no_ln else p(t["beta"]), p(rec),
              rec.numel())
    grads = (p(t["dout"]), p(t["dWf"]), p(o["dq"]), p(o["dk"]), p(o["dv"]), p(o["deta_logit"]),
             p(o["dgate_logit"]), p(o["dW0"]), p(o["dgamma"]), p(o["dbeta"]), B, H, T, d,
             mode, chunk or 1, torch.cuda.current_stream().cuda_stream)
    if noalloc:
        return ttt.ttt_linear_backward_noalloc(*common, *grads)
    return ttt.ttt_linear_backward(*common, p(ws), ws.numel(), *grads)


@pytest.mark.parametrize("first,second", [
    ((8, 16, 100, "exact", False), (2, 3, 37, "st", True)),
    ((4, 8, 53, "st", True), (1, 2, 17, "exact", False)),
    ((2, 4, 40, "none", False), (1, 1, 5, "st", False)),
])
def test_noalloc_backward_matches_workspace_backward(first, second):
    for n, (B, H, T, ln, bf16) in enumerate((first, second)):
        say(f"case no-alloc backward call {n + 1}: B={B} H={H} T={T} ln={ln} bf16={bf16}")
        x, t, rec = setup(B, H, T, ln, bf16, seed=700 + 10 * n + B)
        st, nws = ttt.ttt_linear_backward_workspace_bytes(B, H, 64, ttt.mode_bits(ln))
        assert st == ttt.TTT_OK and nws <= ttt.TTT_STATIC_SCRATCH_BYTES
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        ref, got = outputs(B, H, T, ln), outputs(B, H, T, ln)
        assert call(False, t, rec, ref, B, H, T, ln, bf16, ws) == ttt.TTT_OK
        assert call(True, t, rec, got, B, H, T, ln, bf16) == ttt.TTT_OK
        torch.cuda.synchronize()
        for key in GRADS:
            if ref[key] is None:
                continue
            assert torch.isfinite(ref[key]).all(), key
            assert torch.equal(got[key], ref[key]), key


def test_noalloc_backward_at_its_largest_size():
    # 4096 scans at d = 64 fill the static scratch exactly
    B, H, T = 64, 64, 3
    say(f"case no-alloc backward at the scratch limit: B={B} H={H} T={T}")
    st, nws = ttt.ttt_linear_backward_workspace_bytes(B, H, 64, 0)
    assert st == ttt.TTT_OK and nws == ttt.TTT_STATIC_SCRATCH_BYTES
    x, t, rec = setup(B, H, T, "st", False, seed=790)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ref, got = outputs(B, H, T, "st"), outputs(B, H, T, "st")
    assert call(False, t, rec, ref, B, H, T, "st", False, ws) == ttt.TTT_OK
    assert call(True, t, rec, got, B, H, T, "st", False) == ttt.TTT_OK
    torch.cuda.synchronize()
    for key in GRADS:
        assert torch.isfinite(ref[key]).all(), key
        assert torch.equal(got[key], ref[key]), key


def test_noalloc_backward_vector_alu_kernel():
    # the vector-ALU backward (d other than 64, a dual chunk other than 16)
    # through the same static scratch, two calls in a row, the second smaller
    cases = ((4, 8, 70, "exact", False, 32, 5), (2, 3, 21, "st", True, 16, None))
    for n, (B, H, T, ln, bf16, d, chunk) in enumerate(cases):
        say(f"case no-alloc vector-ALU backward call {n + 1}: B={B} H={H} T={T} ln={ln} "
            f"bf16={bf16} d={d} chunk={chunk}")
        mode = ttt.mode_bits(ln, chunk is not None, bf16)
        assert ttt.ttt_linear_backward_kernel(d, mode, chunk or 1) == "bwd_valu"
        x, t, rec = setup(B, H, T, ln, bf16, seed=800 + n, d=d, chunk=chunk)
        st, nws = ttt.ttt_linear_backward_workspace_bytes(B, H, d, mode)
        assert st == ttt.TTT_OK and nws <= ttt.TTT_STATIC_SCRATCH_BYTES
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        ref, got = outputs(B, H, T, ln, d), outputs(B, H, T, ln, d)
        assert call(False, t, rec, ref, B, H, T, ln, bf16, ws, d=d, chunk=chunk) == ttt.TTT_OK
        assert call(True, t, rec, got, B, H, T, ln, bf16, d=d, chunk=chunk) == ttt.TTT_OK
        torch.cuda.synchronize()
        for key in GRADS:
            assert torch.isfinite(ref[key]).all(), key
            assert torch.equal(got[key], ref[key]), key
