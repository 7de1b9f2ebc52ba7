"""Host-only checks of the C ABI: the library loads, exports what the header
declares, and rejects every invalid argument before touching the GPU.

The checks go through ``ttt_linear_validate``, which runs the same argument
checks as ``ttt_linear_forward`` and never launches; the fake addresses are
never dereferenced.  Where no device is visible, each rejected call is also
sent to ``ttt_linear_forward`` to confirm it returns the same code.
"""
import os
import re
import subprocess

import pytest

import test_rnn_layer_ttt_amd as ttt
from test_rnn_layer_ttt_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_linear.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_\w+)\s*\(", text)))


def header_constants():
    return dict((m, int(v.rstrip("u"))) for m, v in
                re.findall(r"#define\s+(TTT_\w+)\s+(\d+u?)", open(HEADER).read()))


def test_library_exports_every_declared_symbol():
    lib = ttt.load_library()
    declared = header_functions()
    assert declared == sorted(binding.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                        stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r" T (ttt_\w+)", nm))
    assert set(declared) <= exported


def test_binding_constants_match_header():
    for name, value in header_constants().items():
        assert getattr(binding, name) == value, name


def test_version_and_status_strings():
    assert "ttt_linear" in ttt.ttt_version()
    # the library carries the digest of the sources it was built from
    from test_rnn_layer_ttt_amd.build import source_digest
    assert ttt.ttt_version().endswith("src=" + source_digest())
    for code in range(8):
        assert ttt.ttt_status_string(code)
    assert ttt.ttt_status_string(99) == "unknown status"


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# A valid-looking argument set; the tests below break one thing at a time.
_GPU = _gpu_visible()
A = 0x10000000          # 16-byte aligned fake addresses, far apart
STRIDE = 0x10000000


def args(**over):
    base = dict(q=A, k=A + STRIDE, v=A + 2 * STRIDE, eta_logit=A + 3 * STRIDE,
                gate_logit=A + 4 * STRIDE, W0=A + 5 * STRIDE, gamma=A + 6 * STRIDE,
                beta=A + 7 * STRIDE, out=A + 8 * STRIDE, W_final=A + 9 * STRIDE,
                B=2, H=3, T=5, d=64, mode=0, chunk=16, stream=None)
    base.update(over)
    return base


def call(**over):
    """The status ttt_linear_validate returns; where no device is visible, also
    check that ttt_linear_forward returns the same code for the same defect."""
    a = args(**over)
    pos = [a[n] for n in ("q", "k", "v", "eta_logit", "gate_logit", "W0", "gamma", "beta",
                          "out", "W_final", "B", "H", "T", "d", "mode", "chunk")]
    st = ttt.ttt_linear_validate(*pos)
    if st != ttt.TTT_OK and not _GPU:
        assert ttt.ttt_linear_forward(*pos, a["stream"]) == st
    return st


@pytest.mark.parametrize("field", ["q", "k", "v", "eta_logit", "gate_logit", "W0", "gamma",
                                   "beta", "out"])
def test_null_pointer(field):
    assert call(**{field: None, "d": 48}) in (ttt.TTT_ERR_NULL,)


def test_null_gamma_allowed_without_ln_but_other_checks_still_run():
    # NO_LN with gamma=beta=NULL passes the null check and then fails on d
    assert call(gamma=None, beta=None, mode=ttt.TTT_NO_LN, d=48) == ttt.TTT_ERR_UNSUPPORTED


@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(d=0), dict(T=-1), dict(B=-3),
                                  dict(B=1 << 40, H=1 << 40),
                                  dict(B=1 << 20, H=1 << 20, T=1 << 30),
                                  dict(B=1, H=1, T=1 << 62), dict(d=1 << 40)])
def test_bad_shape(over):
    assert call(**over) == ttt.TTT_ERR_SHAPE


@pytest.mark.parametrize("mode", [128, 1 << 10, 0x80000000, ttt.TTT_LN_EXACT | ttt.TTT_NO_LN])
def test_bad_mode(mode):
    assert call(mode=mode) == ttt.TTT_ERR_MODE


@pytest.mark.parametrize("chunk", [0, -5])
def test_dual_needs_positive_chunk(chunk):
    assert call(mode=ttt.TTT_DUAL, chunk=chunk) == ttt.TTT_ERR_MODE


def test_chunk_ignored_without_dual():
    # chunk is not read in per-token mode: the call fails on d, not on chunk
    assert call(chunk=0, d=48) == ttt.TTT_ERR_UNSUPPORTED


@pytest.mark.parametrize("d", [1, 8, 48, 96, 256])
def test_unsupported_d(d):
    assert call(d=d) == ttt.TTT_ERR_UNSUPPORTED


@pytest.mark.parametrize("field,off", [("q", 4), ("k", 8), ("v", 2), ("gate_logit", 12),
                                       ("out", 4), ("W0", 8), ("W_final", 4),
                                       ("eta_logit", 2), ("gamma", 2)])
def test_misaligned(field, off):
    assert call(**{field: args()[field] + off}) == ttt.TTT_ERR_UNSUPPORTED


def test_bf16_eta_needs_only_two_byte_alignment():
    # 2-byte aligned eta passes alignment in bf16 mode; the alias below then trips
    a = args()
    st = call(eta_logit=a["eta_logit"] + 2, mode=ttt.TTT_IN_BF16, out=a["q"])
    assert st == ttt.TTT_ERR_ALIAS


@pytest.mark.parametrize("over", [
    dict(out=A),                          # out == q
    dict(out=A + 2 * STRIDE + 64),        # out inside v
    dict(out=A + 5 * STRIDE),             # out == W0
    dict(W_final=A + 8 * STRIDE),         # W_final == out
    dict(W_final=A + 5 * STRIDE + 256),   # W_final partially overlaps W0
    dict(W_final=A + 3 * STRIDE),         # W_final over eta
    dict(W_final=A + 6 * STRIDE),         # W_final over gamma
])
def test_alias_rejected(over):
    assert call(**over) == ttt.TTT_ERR_ALIAS


def test_inputs_may_alias_each_other_and_state_in_place():
    a = args()
    assert call(k=a["q"], v=a["q"], W_final=a["W0"]) == ttt.TTT_OK
    assert call(W_final=None) == ttt.TTT_OK
    assert call(gamma=None, beta=None, mode=ttt.TTT_NO_LN) == ttt.TTT_OK


def test_empty_sequence_allows_null_sequence_pointers():
    st = call(q=None, k=None, v=None, eta_logit=None, gate_logit=None, out=None, T=0)
    assert st == ttt.TTT_OK


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("mode", [0, 1, 2, 4, 8, 5, 7, 13, 16, 23, 29, 32, 37, 55, 61])
def test_supported_combinations_validate(d, mode):
    assert call(d=d, mode=mode) == ttt.TTT_OK


def test_kernel_choice():
    # d = 64 runs on the matrix cores (per-token, and the dual form with chunks of 16) ...
    assert ttt.ttt_linear_kernel(64, 0, 1) == "scan_mfma"
    assert ttt.ttt_linear_kernel(64, ttt.TTT_DUAL | ttt.TTT_IN_BF16, 16) == "scan_mfma"
    assert ttt.ttt_linear_kernel(64, ttt.TTT_DUAL, 8) == "scan_valu"
    # ... unless the vector-ALU kernel is asked for
    assert ttt.ttt_linear_kernel(64, ttt.TTT_FORCE_VALU, 1) == "scan_valu"
    assert ttt.ttt_linear_kernel(64, ttt.TTT_FORCE_VALU | ttt.TTT_DUAL, 16) == "scan_valu"
    for d in (16, 32, 128):
        assert ttt.ttt_linear_kernel(d, 0, 1) == "scan_valu"
    assert ttt.ttt_linear_kernel(48, 0, 1) == "none"


def test_stale_library_is_refused(tmp_path, monkeypatch):
    # a library whose digest does not match the sources must not load
    from test_rnn_layer_ttt_amd import build as build_mod
    monkeypatch.setattr(build_mod, "source_digest", lambda kernel=None: "0" * 16)
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="stale"):
        binding.load_library()
    monkeypatch.undo()
    binding._lib = None
    assert binding.load_library() is not None


def test_error_codes_raise_from_check():
    with pytest.raises(ValueError):
        binding.check(ttt.TTT_ERR_SHAPE)
    with pytest.raises(RuntimeError):
        binding.check(ttt.TTT_ERR_HIP)
    binding.check(ttt.TTT_OK)


def test_mode_bits():
    assert ttt.mode_bits() == 0
    assert ttt.mode_bits("exact", True, True) == ttt.TTT_LN_EXACT | ttt.TTT_DUAL | ttt.TTT_IN_BF16
    assert ttt.mode_bits("none") == ttt.TTT_NO_LN
    assert ttt.mode_bits(force_valu=True) == ttt.TTT_FORCE_VALU
    with pytest.raises(ValueError):
        ttt.mode_bits("bogus")
