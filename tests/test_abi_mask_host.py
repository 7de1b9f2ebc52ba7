"""Host-only checks of ttt_linear_forward_masked's own argument rules (the
forward's rules run first and are covered in test_abi_host).  Rejected calls
launch nothing; they are sent only where no device is visible."""
import pytest

import test_rnn_layer_ttt_amd as ttt

from .test_abi_host import _GPU

A = 0x10000000
S = 0x10000000

pytestmark = pytest.mark.skipif(_GPU, reason="sends unlaunchable arguments to an entry point")


def call(**over):
    a = dict(q=A, k=A + S, v=A + 2 * S, eta_logit=A + 3 * S, gate_logit=A + 4 * S, W0=A + 5 * S,
             gamma=A + 6 * S, beta=A + 7 * S, update_mask=A + 10 * S, out=A + 8 * S,
             W_final=A + 9 * S, B=2, H=3, T=37, d=64, mode=ttt.TTT_DUAL, chunk=16, stream=None)
    a.update(over)
    return ttt.ttt_linear_forward_masked(*a.values())


def test_needs_dual():
    assert call(mode=0) == ttt.TTT_ERR_MODE
    assert call(mode=ttt.TTT_LN_EXACT) == ttt.TTT_ERR_MODE


def test_needs_a_mask_when_there_are_tokens():
    assert call(update_mask=None) == ttt.TTT_ERR_NULL


def test_empty_sequence_needs_no_mask():
    # no W_final and T == 0: nothing to launch or copy
    st = call(update_mask=None, T=0, W_final=None, q=None, k=None, v=None, eta_logit=None,
              gate_logit=None, out=None)
    assert st == ttt.TTT_OK


@pytest.mark.parametrize("where", [A + 8 * S, A + 8 * S + 1000, A + 9 * S + 5])
def test_mask_must_not_overlap_outputs(where):
    assert call(update_mask=where) == ttt.TTT_ERR_ALIAS


def test_mask_may_alias_inputs_and_needs_no_alignment():
    # the mask is read-only like the inputs; a byte array needs no alignment.
    # The call then passes validation; without a device the launch fails.
    st = call(update_mask=A + 2 * S + 3)
    assert st == ttt.TTT_ERR_HIP


def test_forward_checks_come_first():
    assert call(d=48) == ttt.TTT_ERR_UNSUPPORTED
    assert call(out=A) == ttt.TTT_ERR_ALIAS
    assert call(chunk=0) == ttt.TTT_ERR_MODE
