"""Host-only checks of the training entry points of the C ABI: the record and
workspace size queries, and the argument checks of the recording forward and
of the backward.

Every check runs before the first HIP call.  The rejected calls below are sent
to the real entry points only where no device is visible (the fake addresses
are never dereferenced, and a rejected call launches nothing).
"""
import pytest

import test_rnn_layer_ttt_amd as ttt

from .test_abi_host import _GPU

A = 0x10000000
S = 0x10000000
B, H, T, D = 2, 3, 37, 64


def rec_bytes(B=B, H=H, T=T, d=D, mode=0):
    st, n = ttt.ttt_linear_record_bytes(B, H, T, d, mode)
    assert st == ttt.TTT_OK
    return n


@pytest.mark.parametrize("B_,H_,T_", [(1, 1, 0), (1, 1, 1), (2, 3, 16), (2, 3, 17), (4, 32, 16384)])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_record_bytes_formula(B_, H_, T_, d):
    ntiles = -(-T_ // 16)
    assert rec_bytes(B_, H_, T_, d) == 4 * B_ * H_ * (T_ * d + ntiles * d * d)


def ws_bytes(B=B, H=H, d=D, mode=0):
    st, n = ttt.ttt_linear_backward_workspace_bytes(B, H, d, mode)
    assert st == ttt.TTT_OK
    return n


@pytest.mark.parametrize("mode", [0, ttt.TTT_LN_EXACT, ttt.TTT_IN_BF16, ttt.TTT_DUAL,
                                  ttt.TTT_SILU_QK])
def test_workspace_bytes_formula(mode):
    # per (b,h): dgamma and dbeta before their sum over the batch
    assert ws_bytes(B, H, D, mode) == 4 * B * H * 2 * 64
    assert ws_bytes(B, H, D, (mode & ~ttt.TTT_LN_EXACT) | ttt.TTT_NO_LN) == 0
    assert ws_bytes(B, H, 16, mode) == 4 * B * H * 2 * 16


@pytest.mark.parametrize("over,code", [
    (dict(d=48), ttt.TTT_ERR_UNSUPPORTED),
    (dict(d=256), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=1 << 10), ttt.TTT_ERR_MODE),
    (dict(B=0), ttt.TTT_ERR_SHAPE),
])
def test_workspace_bytes_rejects(over, code):
    a = dict(B=B, H=H, d=D, mode=0)
    a.update(over)
    assert ttt.ttt_linear_backward_workspace_bytes(a["B"], a["H"], a["d"], a["mode"])[0] == code


@pytest.mark.parametrize("mode", [0, ttt.TTT_LN_EXACT, ttt.TTT_NO_LN, ttt.TTT_IN_BF16,
                                  ttt.TTT_IN_BF16 | ttt.TTT_LN_EXACT, ttt.TTT_DUAL,
                                  ttt.TTT_DUAL | ttt.TTT_IN_BF16 | ttt.TTT_NO_LN,
                                  ttt.TTT_DUAL | ttt.TTT_SILU_QK])
def test_record_bytes_independent_of_dtype_ln_and_form(mode):
    assert rec_bytes(mode=mode) == rec_bytes()


@pytest.mark.parametrize("over,code", [
    (dict(d=48), ttt.TTT_ERR_UNSUPPORTED),
    (dict(d=8), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=1 << 10), ttt.TTT_ERR_MODE),
    (dict(mode=ttt.TTT_LN_EXACT | ttt.TTT_NO_LN), ttt.TTT_ERR_MODE),
    (dict(B=0), ttt.TTT_ERR_SHAPE),
    (dict(T=-1), ttt.TTT_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 20, T=1 << 30), ttt.TTT_ERR_SHAPE),
    (dict(T=1 << 60), ttt.TTT_ERR_SHAPE),
])
def test_record_bytes_rejects(over, code):
    a = dict(B=B, H=H, T=T, d=D, mode=0)
    a.update(over)
    assert ttt.ttt_linear_record_bytes(a["B"], a["H"], a["T"], a["d"], a["mode"])[0] == code


# ---------------------------------------------------------------------------
# recording forward
# ---------------------------------------------------------------------------
def fwd_args(**over):
    base = dict(q=A, k=A + S, v=A + 2 * S, eta_logit=A + 3 * S, gate_logit=A + 4 * S,
                W0=A + 5 * S, gamma=A + 6 * S, beta=A + 7 * S, out=A + 8 * S, W_final=A + 9 * S,
                record=A + 10 * S, record_bytes=rec_bytes(), B=B, H=H, T=T, d=D, mode=0,
                chunk=16, stream=None)
    base.update(over)
    return base


def fwd_call(**over):
    a = fwd_args(**over)
    return ttt.ttt_linear_forward_record(*a.values())


needs_no_gpu = pytest.mark.skipif(_GPU, reason="sends unlaunchable arguments to an entry point")


@needs_no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(record=None), ttt.TTT_ERR_NULL),
    (dict(record=A + 10 * S + 8), ttt.TTT_ERR_UNSUPPORTED),
    (dict(record_bytes=rec_bytes() - 1), ttt.TTT_ERR_WORKSPACE),
    (dict(record_bytes=0), ttt.TTT_ERR_WORKSPACE),
    (dict(record=A + 8 * S), ttt.TTT_ERR_ALIAS),            # record == out
    (dict(record=A + 2 * S + 4096), ttt.TTT_ERR_ALIAS),     # record inside v
    (dict(record=A + 9 * S), ttt.TTT_ERR_ALIAS),            # record == W_final
    (dict(record=A + 5 * S), ttt.TTT_ERR_ALIAS),            # record == W0
    (dict(mode=ttt.TTT_DUAL, chunk=0), ttt.TTT_ERR_MODE),
    (dict(d=48), ttt.TTT_ERR_UNSUPPORTED),
    (dict(q=None), ttt.TTT_ERR_NULL),                       # the forward's own checks first
    (dict(out=A), ttt.TTT_ERR_ALIAS),
    (dict(mode=ttt.TTT_LN_EXACT | ttt.TTT_NO_LN), ttt.TTT_ERR_MODE),
    # any chunk, d and the vector-ALU kernel record too: these reach the record's checks
    (dict(mode=ttt.TTT_DUAL, chunk=8, record_bytes=1), ttt.TTT_ERR_WORKSPACE),
    (dict(mode=ttt.TTT_DUAL, chunk=100, record_bytes=1), ttt.TTT_ERR_WORKSPACE),
    (dict(d=16, record_bytes=rec_bytes(d=16) - 4), ttt.TTT_ERR_WORKSPACE),
    (dict(mode=ttt.TTT_FORCE_VALU, record=A + 8 * S), ttt.TTT_ERR_ALIAS),
])
def test_forward_record_rejects(over, code):
    assert fwd_call(**over) == code


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
BWD_FIELDS = ("q", "k", "v", "eta_logit", "gate_logit", "gamma", "beta", "record",
              "record_bytes", "workspace", "workspace_bytes", "dout", "dW_final", "dq", "dk", "dv", "deta_logit", "dgate_logit",
              "dW0", "dgamma", "dbeta", "B", "H", "T", "d", "mode", "chunk", "stream")


def bwd_args(**over):
    names = ("q", "k", "v", "eta_logit", "gate_logit", "gamma", "beta", "record", None, "dout",
             "dW_final", "dq", "dk", "dv", "deta_logit", "dgate_logit", "dW0", "dgamma", "dbeta")
    base = {n: A + i * S for i, n in enumerate(names) if n is not None}
    base.update(record_bytes=rec_bytes(), workspace=A + 19 * S, workspace_bytes=ws_bytes(),
                B=B, H=H, T=T, d=D, mode=0, chunk=16, stream=None)
    base.update(over)
    return base


def bwd_call(**over):
    a = bwd_args(**over)
    return ttt.ttt_linear_backward(*[a[f] for f in BWD_FIELDS])


@needs_no_gpu
@pytest.mark.parametrize("field", ["q", "k", "v", "eta_logit", "gate_logit", "gamma", "beta",
                                   "record", "dout", "dq", "dk", "dv", "deta_logit",
                                   "dgate_logit", "dW0", "dgamma", "dbeta"])
def test_backward_null(field):
    assert bwd_call(**{field: None}) == ttt.TTT_ERR_NULL


@needs_no_gpu
@pytest.mark.parametrize("field", ["q", "dout", "dq", "dk", "dv", "dgate_logit", "dW0",
                                   "dW_final", "record", "workspace"])
def test_backward_misaligned(field):
    assert bwd_call(**{field: bwd_args()[field] + 4}) == ttt.TTT_ERR_UNSUPPORTED


@needs_no_gpu
def test_backward_eta_alignment_follows_dtype():
    a = bwd_args()
    assert bwd_call(eta_logit=a["eta_logit"] + 2) == ttt.TTT_ERR_UNSUPPORTED
    assert bwd_call(deta_logit=a["deta_logit"] + 2) == ttt.TTT_ERR_UNSUPPORTED
    # bf16: 2-byte eta passes alignment; dq == q then trips the alias check
    assert bwd_call(eta_logit=a["eta_logit"] + 2, mode=ttt.TTT_IN_BF16,
                    dq=a["q"]) == ttt.TTT_ERR_ALIAS


@needs_no_gpu
@pytest.mark.parametrize("over", [
    dict(dq=A),                    # dq == q
    dict(dk=A + 11 * S),           # dk == dq
    dict(dv=A + 11 * S + 256),     # dv inside dq
    dict(dW0=A + 10 * S + 64),     # dW0 partially over dW_final
    dict(dgamma=A + 5 * S),        # dgamma == gamma
    dict(dbeta=A + 17 * S),        # dbeta == dgamma
    dict(record=A + 17 * S),       # record == dgamma
    dict(deta_logit=A + 7 * S + 1024),   # deta inside the record (an input)
    dict(record=A + 11 * S),       # record == dq
    dict(workspace=A + 7 * S),     # workspace == record
    dict(workspace=A + 11 * S + 512),    # workspace inside dq
    dict(workspace=A + 18 * S),    # workspace == dbeta
    dict(workspace=A + 5 * S),     # workspace == gamma
])
def test_backward_alias_rejected(over):
    assert bwd_call(**over) == ttt.TTT_ERR_ALIAS


@needs_no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(mode=ttt.TTT_DUAL, chunk=8, record_bytes=1), ttt.TTT_ERR_WORKSPACE),
    (dict(mode=ttt.TTT_DUAL, chunk=1, workspace_bytes=0), ttt.TTT_ERR_WORKSPACE),
    (dict(mode=ttt.TTT_DUAL, chunk=0), ttt.TTT_ERR_MODE),
    (dict(d=48), ttt.TTT_ERR_UNSUPPORTED),
    (dict(d=16, record_bytes=rec_bytes(d=16) - 4), ttt.TTT_ERR_WORKSPACE),
    (dict(record_bytes=rec_bytes() - 4), ttt.TTT_ERR_WORKSPACE),
    (dict(workspace_bytes=ws_bytes() - 4), ttt.TTT_ERR_WORKSPACE),
    (dict(workspace_bytes=0), ttt.TTT_ERR_WORKSPACE),
    (dict(workspace=None), ttt.TTT_ERR_NULL),
    (dict(mode=1 << 10), ttt.TTT_ERR_MODE),
    (dict(H=0), ttt.TTT_ERR_SHAPE),
])
def test_backward_rejects(over, code):
    assert bwd_call(**over) == code


@needs_no_gpu
def test_backward_without_ln_ignores_affine_pointers():
    # NO_LN: gamma, beta, dgamma, dbeta may be NULL; the record size check still runs
    st = bwd_call(gamma=None, beta=None, dgamma=None, dbeta=None, mode=ttt.TTT_NO_LN,
                  record_bytes=1)
    assert st == ttt.TTT_ERR_WORKSPACE
    # ... and the workspace is not needed at all
    st = bwd_call(gamma=None, beta=None, dgamma=None, dbeta=None, mode=ttt.TTT_NO_LN,
                  workspace=None, workspace_bytes=0, record_bytes=1)
    assert st == ttt.TTT_ERR_WORKSPACE


@needs_no_gpu
def test_backward_empty_sequence_allows_null_token_pointers():
    st = bwd_call(q=None, k=None, v=None, eta_logit=None, gate_logit=None, dout=None, dq=None,
                  dk=None, dv=None, deta_logit=None, dgate_logit=None, T=0,
                  record_bytes=rec_bytes(T=0) - 1)
    assert st == ttt.TTT_ERR_WORKSPACE
    # the record of an empty sequence is empty and may be NULL (the check that
    # trips is then the workspace size, after the pointer checks)
    assert rec_bytes(T=0) == 0
    st = bwd_call(q=None, k=None, v=None, eta_logit=None, gate_logit=None, dout=None, dq=None,
                  dk=None, dv=None, deta_logit=None, dgate_logit=None, T=0, record=None,
                  record_bytes=0, workspace_bytes=0)
    assert st == ttt.TTT_ERR_WORKSPACE
    assert bwd_call(T=1, record=None) == ttt.TTT_ERR_NULL


@needs_no_gpu
def test_noalloc_backward_checks_like_the_backward_and_bounds_its_scratch():
    names = [f for f in BWD_FIELDS if f not in ("workspace", "workspace_bytes")]
    nb = lambda **over: ttt.ttt_linear_backward_noalloc(*[bwd_args(**over)[f] for f in names])
    # the argument checks of the backward ...
    assert nb(dq=None) == ttt.TTT_ERR_NULL
    assert nb(dq=A) == ttt.TTT_ERR_ALIAS
    assert nb(d=48) == ttt.TTT_ERR_UNSUPPORTED
    assert nb(mode=ttt.TTT_DUAL, chunk=0) == ttt.TTT_ERR_MODE
    # ... and the static scratch's bound: 4096 scans at d = 64 fit, 4097 do not
    assert ttt.TTT_STATIC_SCRATCH_BYTES == 2 * 1024 * 1024
    big = dict(B=4097, H=1, T=1, record_bytes=rec_bytes(4097, 1, 1))
    assert nb(**big) == ttt.TTT_ERR_WORKSPACE
    big = dict(B=64, H=65, T=2, record_bytes=rec_bytes(64, 65, 2))
    assert nb(**big) == ttt.TTT_ERR_WORKSPACE
    # without the LayerNorm there is no scratch, so any size passes that check
    # (and then stops at the size of the record)
    assert nb(B=64, H=65, T=2, gamma=None, beta=None, dgamma=None, dbeta=None,
              mode=ttt.TTT_NO_LN, record_bytes=1) == ttt.TTT_ERR_WORKSPACE
    assert nb(B=64, H=65, T=2, record_bytes=1) == ttt.TTT_ERR_WORKSPACE


def test_status_string_of_workspace_error():
    s = ttt.ttt_status_string(ttt.TTT_ERR_WORKSPACE)
    assert "record" in s and "workspace" in s


@pytest.mark.parametrize("d,mode,chunk,kernel", [
    (64, 0, 1, "bwd_mfma"),
    (64, ttt.TTT_LN_EXACT | ttt.TTT_IN_BF16, 1, "bwd_mfma"),
    (64, ttt.TTT_DUAL, 16, "bwd_mfma"),
    (64, ttt.TTT_DUAL, 8, "bwd_valu"),
    (64, ttt.TTT_DUAL, 32, "bwd_valu"),
    (64, ttt.TTT_FORCE_VALU, 1, "bwd_valu"),
    (16, 0, 1, "bwd_valu"),
    (32, ttt.TTT_NO_LN, 1, "bwd_valu"),
    (128, ttt.TTT_DUAL | ttt.TTT_LN_EXACT, 5, "bwd_valu"),
    (48, 0, 1, "none"),
    (64, ttt.TTT_DUAL, 0, "none"),
    (64, ttt.TTT_LN_EXACT | ttt.TTT_NO_LN, 1, "none"),
])
def test_backward_kernel_routing(d, mode, chunk, kernel):
    assert ttt.ttt_linear_backward_kernel(d, mode, chunk) == kernel
