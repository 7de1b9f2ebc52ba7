"""Host-only checks of the input-projection entry point of the C ABI
(``ttt_linear_project``): every argument rule, before any HIP call.  The
rejected calls are sent to the real entry point only where no device is
visible (the fake addresses are never dereferenced, and a rejected call
launches nothing)."""
import pytest

import test_rnn_layer_ttt_amd as ttt

from .test_abi_host import _GPU

A = 0x10000000
S = 0x10000000
B, T, HID, H, D = 2, 37, 128, 3, 64
FIELDS = ("x", "w_proj", "b_proj", "q", "k", "v", "eta_logit", "gate_logit", "B", "T",
          "hidden", "H", "d", "mode", "stream")


def args(**over):
    base = {n: A + i * S for i, n in enumerate(FIELDS[:8])}
    base.update(B=B, T=T, hidden=HID, H=H, d=D, mode=ttt.TTT_IN_BF16, stream=None)
    base.update(over)
    return base


def call(**over):
    a = args(**over)
    return ttt.ttt_linear_project(*[a[f] for f in FIELDS])


needs_no_gpu = pytest.mark.skipif(_GPU, reason="sends unlaunchable arguments to an entry point")


@needs_no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(mode=1 << 10), ttt.TTT_ERR_MODE),
    (dict(B=0), ttt.TTT_ERR_SHAPE),
    (dict(H=0), ttt.TTT_ERR_SHAPE),
    (dict(hidden=0), ttt.TTT_ERR_SHAPE),
    (dict(T=-1), ttt.TTT_ERR_SHAPE),
    (dict(B=1 << 40, T=1 << 40), ttt.TTT_ERR_SHAPE),
    (dict(d=32), ttt.TTT_ERR_UNSUPPORTED),
    (dict(hidden=48), ttt.TTT_ERR_UNSUPPORTED),   # not a multiple of 32
    (dict(hidden=65536 + 32), ttt.TTT_ERR_UNSUPPORTED),   # beyond 32-bit lane offsets
    (dict(T=1 << 33), ttt.TTT_ERR_UNSUPPORTED),   # T beyond 32 bits
    (dict(B=1 << 20, T=1 << 30), ttt.TTT_ERR_UNSUPPORTED),   # more workgroups than a launch takes
    (dict(x=None), ttt.TTT_ERR_NULL),
    (dict(w_proj=None), ttt.TTT_ERR_NULL),
    (dict(eta_logit=None), ttt.TTT_ERR_NULL),
    (dict(x=A + 8), ttt.TTT_ERR_UNSUPPORTED),
    (dict(w_proj=A + S + 2), ttt.TTT_ERR_UNSUPPORTED),
    (dict(q=A + 3 * S + 4), ttt.TTT_ERR_UNSUPPORTED),
    (dict(b_proj=A + 2 * S + 2), ttt.TTT_ERR_UNSUPPORTED),
    (dict(eta_logit=A + 6 * S + 2, mode=0), ttt.TTT_ERR_UNSUPPORTED),   # fp32 eta needs 4
    (dict(k=A + 3 * S), ttt.TTT_ERR_ALIAS),                  # k == q
    (dict(q=A), ttt.TTT_ERR_ALIAS),                          # q == x
    (dict(gate_logit=A + 6 * S + 64), ttt.TTT_ERR_ALIAS),    # gate over eta
    (dict(b_proj=A + 5 * S), ttt.TTT_ERR_ALIAS),             # bias inside v
    (dict(v=A + S + 4096), ttt.TTT_ERR_ALIAS),               # v inside w_proj
])
def test_project_rejects(over, code):
    assert call(**over) == code


@needs_no_gpu
def test_bf16_eta_needs_only_two_byte_alignment():
    # passes alignment with bf16 outputs; q == x then trips the alias check
    assert call(eta_logit=A + 6 * S + 2, q=A) == ttt.TTT_ERR_ALIAS


def test_empty_sequence_is_a_no_op_with_null_pointers():
    st = ttt.ttt_linear_project(None, None, None, None, None, None, None, None, 2, 0, 128, 3,
                                64, ttt.TTT_IN_BF16, None)
    assert st == ttt.TTT_OK


@needs_no_gpu
def test_hidden_65536_is_supported():
    # passes the size rules; q == x then trips the alias check
    assert call(hidden=65536, q=A) == ttt.TTT_ERR_ALIAS


def test_bias_is_optional():
    # a NULL bias is no error: the rest of the checks decide (here: the alias)
    assert call(b_proj=None, q=A) == ttt.TTT_ERR_ALIAS
