"""Host-only checks of the two-layer scan's C entry points: every invalid
argument of ``ttt_mlp_forward`` is rejected by ``ttt_mlp_validate`` (the same
checks, no launch; the fake addresses are never dereferenced), and the kernel
query names the kernel each mode runs."""
import pytest

import test_rnn_layer_ttt_amd as ttt

A = 0x10000000          # 16-byte aligned fake addresses, far apart
S = 0x10000000
NAMES = ("q", "k", "v", "eta_logit", "gate_logit", "W1_0", "W2_0", "gamma", "beta", "out",
         "W1_final", "W2_final", "B", "H", "T", "d", "mode", "chunk")


def call(**over):
    a = dict(zip(NAMES[:12], [A + i * S for i in range(12)]))
    a.update(B=2, H=3, T=5, d=64, mode=0, chunk=16)
    a.update(over)
    return ttt.ttt_mlp_validate(*[a[n] for n in NAMES])


def test_valid_call_passes():
    assert call() == ttt.TTT_OK
    for d in (16, 32, 64):
        assert call(d=d) == ttt.TTT_OK
    for mode in (ttt.TTT_DUAL, ttt.TTT_LN_EXACT, ttt.TTT_NO_LN, ttt.TTT_IN_BF16,
                 ttt.TTT_FORCE_VALU, ttt.TTT_DUAL | ttt.TTT_IN_BF16 | ttt.TTT_LN_EXACT):
        assert call(mode=mode) == ttt.TTT_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "eta_logit", "gate_logit", "W1_0", "W2_0",
                                   "gamma", "beta", "out"])
def test_null_pointer(field):
    assert call(**{field: None}) == ttt.TTT_ERR_NULL


def test_nulls_allowed():
    assert call(W1_final=None, W2_final=None) == ttt.TTT_OK
    assert call(gamma=None, beta=None, mode=ttt.TTT_NO_LN) == ttt.TTT_OK
    # an empty sequence reads and writes no sequence array
    assert call(T=0, q=None, k=None, v=None, eta_logit=None, gate_logit=None,
                out=None) == ttt.TTT_OK


@pytest.mark.parametrize("over,status", [
    (dict(B=0), ttt.TTT_ERR_SHAPE), (dict(T=-1), ttt.TTT_ERR_SHAPE),
    (dict(d=128), ttt.TTT_ERR_UNSUPPORTED), (dict(d=48), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=ttt.TTT_SILU_QK), ttt.TTT_ERR_UNSUPPORTED),
    (dict(mode=128), ttt.TTT_ERR_MODE), (dict(mode=ttt.TTT_LN_EXACT | ttt.TTT_NO_LN),
                                         ttt.TTT_ERR_MODE),
    (dict(mode=ttt.TTT_DUAL, chunk=0), ttt.TTT_ERR_MODE),
    (dict(W2_0=A + 6 * S + 8), ttt.TTT_ERR_UNSUPPORTED),
    (dict(W2_final=A + 11 * S + 4), ttt.TTT_ERR_UNSUPPORTED),
    (dict(W1_0=A + 5 * S + 8), ttt.TTT_ERR_UNSUPPORTED),
])
def test_rejected(over, status):
    assert call(**over) == status


W = 2 * 3 * 64 * 64 * 4   # bytes of one weight at the default sizes


@pytest.mark.parametrize("over", [
    dict(W2_final=A),                      # onto q
    dict(W2_final=A + 5 * S),              # onto W1_0
    dict(W2_final=A + 9 * S),              # onto out
    dict(W2_final=A + 10 * S),             # onto W1_final
    dict(W2_final=A + 6 * S + W // 2),     # part of W2_0
    dict(W2_0=A + 9 * S),                  # W2_0 under out
    dict(W2_0=A + 10 * S),                 # W2_0 under W1_final
    dict(W1_final=A + 6 * S),              # W1_final onto W2_0
    dict(out=A + 6 * S),                   # out onto W2_0
])
def test_aliasing(over):
    assert call(**over) == ttt.TTT_ERR_ALIAS


def test_in_place_states_allowed():
    assert call(W1_final=A + 5 * S, W2_final=A + 6 * S) == ttt.TTT_OK


def test_kernel_query():
    assert ttt.ttt_mlp_kernel(64, ttt.TTT_SILU_QK, 1) == "none"
    assert ttt.ttt_mlp_kernel(128, 0, 1) == "none"
    for d in (16, 32, 64):
        assert ttt.ttt_mlp_kernel(d, 0, 1) == "mlp_valu"
    assert ttt.ttt_mlp_kernel(64, ttt.TTT_FORCE_VALU | ttt.TTT_DUAL | ttt.TTT_IN_BF16,
                              16) == "mlp_valu"
    # the matrix-core kernel: dual form, chunks of 16, bf16 inputs, d = 64, every LN mode
    for ln in (0, ttt.TTT_LN_EXACT, ttt.TTT_NO_LN):
        assert ttt.ttt_mlp_kernel(64, ln | ttt.TTT_DUAL | ttt.TTT_IN_BF16, 16) == "mlp_mfma"
    assert ttt.ttt_mlp_kernel(64, ttt.TTT_DUAL | ttt.TTT_IN_BF16, 8) == "mlp_valu"
    assert ttt.ttt_mlp_kernel(64, ttt.TTT_DUAL, 16) == "mlp_valu"
    assert ttt.ttt_mlp_kernel(32, ttt.TTT_DUAL | ttt.TTT_IN_BF16, 16) == "mlp_valu"
    assert ttt.ttt_mlp_kernel(64, ttt.TTT_IN_BF16, 1) == "mlp_valu"
