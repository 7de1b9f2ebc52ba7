"""Host-only checks of the training entry points of the C ABI: the record size
query, and the argument checks of the recording forward and of the backward.

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
def test_record_bytes_formula(B_, H_, T_):
    ntiles = -(-T_ // 16)
    assert rec_bytes(B_, H_, T_) == 4 * B_ * H_ * (T_ * 64 + ntiles * 64 * 64 + 2 * 64)


@pytest.mark.parametrize("mode", [0, ttt.TTT_LN_EXACT, ttt.TTT_NO_LN, ttt.TTT_IN_BF16,
                                  ttt.TTT_IN_BF16 | ttt.TTT_LN_EXACT, ttt.TTT_DUAL,
                                  ttt.TTT_DUAL | ttt.TTT_IN_BF16 | ttt.TTT_NO_LN,
                                  ttt.TTT_DUAL | ttt.TTT_SILU_QK])
def test_record_bytes_independent_of_dtype_ln_and_form(mode):
    assert rec_bytes(mode=mode) == rec_bytes()


@pytest.mark.parametrize("over,code", [
    (dict(d=32), ttt.TTT_ERR_UNSUPPORTED),
    (dict(d=128), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=32), ttt.TTT_ERR_MODE),
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
    (dict(mode=ttt.TTT_DUAL, chunk=8), ttt.TTT_ERR_UNSUPPORTED),    # chunks must be the tiles
    (dict(mode=ttt.TTT_DUAL, chunk=32), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=ttt.TTT_DUAL, chunk=0), ttt.TTT_ERR_MODE),
    (dict(d=32), ttt.TTT_ERR_UNSUPPORTED),
    (dict(q=None), ttt.TTT_ERR_NULL),                       # the forward's own checks first
    (dict(out=A), ttt.TTT_ERR_ALIAS),
    (dict(mode=ttt.TTT_LN_EXACT | ttt.TTT_NO_LN), ttt.TTT_ERR_MODE),
])
def test_forward_record_rejects(over, code):
    assert fwd_call(**over) == code


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
BWD_FIELDS = ("q", "k", "v", "eta_logit", "gate_logit", "gamma", "beta", "record",
              "record_bytes", "dout", "dW_final", "dq", "dk", "dv", "deta_logit", "dgate_logit",
              "dW0", "dgamma", "dbeta", "B", "H", "T", "d", "mode", "chunk", "stream")


def bwd_args(**over):
    names = ("q", "k", "v", "eta_logit", "gate_logit", "gamma", "beta", "record", None, "dout",
             "dW_final", "dq", "dk", "dv", "deta_logit", "dgate_logit", "dW0", "dgamma", "dbeta")
    base = {n: A + i * S for i, n in enumerate(names) if n is not None}
    base.update(record_bytes=rec_bytes(), B=B, H=H, T=T, d=D, mode=0, chunk=16, stream=None)
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
                                   "dW_final", "record"])
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
    dict(record=A + 9 * S),        # record == dout
    dict(deta_logit=A + 7 * S + 1024),   # deta inside the record
])
def test_backward_alias_rejected(over):
    assert bwd_call(**over) == ttt.TTT_ERR_ALIAS


@needs_no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(mode=ttt.TTT_DUAL, chunk=8), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=ttt.TTT_DUAL, chunk=1), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=ttt.TTT_DUAL, chunk=0), ttt.TTT_ERR_MODE),
    (dict(d=16), ttt.TTT_ERR_UNSUPPORTED),
    (dict(record_bytes=rec_bytes() - 4), ttt.TTT_ERR_WORKSPACE),
    (dict(mode=32), ttt.TTT_ERR_MODE),
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


@needs_no_gpu
def test_backward_empty_sequence_allows_null_token_pointers():
    st = bwd_call(q=None, k=None, v=None, eta_logit=None, gate_logit=None, dout=None, dq=None,
                  dk=None, dv=None, deta_logit=None, dgate_logit=None, T=0,
                  record_bytes=rec_bytes(T=0) - 1)
    assert st == ttt.TTT_ERR_WORKSPACE


def test_status_string_of_workspace_error():
    assert "record" in ttt.ttt_status_string(ttt.TTT_ERR_WORKSPACE)
