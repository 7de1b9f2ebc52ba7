"""Thin ctypes binding of ``libttt_linear.so`` (argument marshalling only).

The functions below carry the names of the C entry points declared in
``include/ttt_linear.h`` and pass raw device pointers, sizes and the HIP
stream straight through; every step of the scan runs in the library's HIP
kernels.  PyTorch is used only to own device memory and to name the current
stream.  If the library has not been built, the first call raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt_linear.so")

# mode bits and status codes, as in include/ttt_linear.h
TTT_DUAL = 1
TTT_LN_EXACT = 2
TTT_IN_BF16 = 4
TTT_NO_LN = 8

TTT_OK = 0
TTT_ERR_NULL = 1
TTT_ERR_SHAPE = 2
TTT_ERR_MODE = 3
TTT_ERR_UNSUPPORTED = 4
TTT_ERR_ALIAS = 5
TTT_ERR_HIP = 6

#: every symbol the header declares
EXPORTED = ("ttt_linear_forward", "ttt_linear_kernel", "ttt_linear_validate",
            "ttt_status_string", "ttt_version")

_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ttt_linear_forward failed with status {status}: {message}")
        self.status = status


class TTTArgumentError(TTTError, ValueError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.ttt_linear_forward.restype = ctypes.c_int32
    lib.ttt_linear_forward.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_linear_validate.restype = ctypes.c_int32
    lib.ttt_linear_validate.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_linear_kernel.restype = ctypes.c_char_p
    lib.ttt_linear_kernel.argtypes = [ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_status_string.argtypes = [ctypes.c_int32]
    lib.ttt_version.restype = ctypes.c_char_p
    lib.ttt_version.argtypes = []
    _lib = lib
    return lib


def ttt_status_string(status: int) -> str:
    return load_library().ttt_status_string(int(status)).decode()


def ttt_linear_kernel(d: int, mode: int, chunk: int) -> str:
    """Name of the kernel family a valid call with these settings launches."""
    return load_library().ttt_linear_kernel(int(d), ctypes.c_uint32(int(mode)), int(chunk)).decode()


def ttt_version() -> str:
    return load_library().ttt_version().decode()


def ttt_linear_forward(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final,
                       B, H, T, d, mode, chunk, stream) -> int:
    """Call the C entry point with raw pointers (ints or None) and sizes.

    Returns the status code unchanged; see :func:`check` to raise on error.
    """
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_forward(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W0), p(gamma), p(beta), p(out),
        p(W_final), int(B), int(H), int(T), int(d), ctypes.c_uint32(int(mode)),
        int(chunk), p(stream)))


def ttt_linear_validate(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final,
                        B, H, T, d, mode, chunk) -> int:
    """Only the argument checks of :func:`ttt_linear_forward`; never launches."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_validate(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W0), p(gamma), p(beta), p(out),
        p(W_final), int(B), int(H), int(T), int(d), ctypes.c_uint32(int(mode)), int(chunk)))


def check(status: int) -> None:
    """Raise for a non-OK status: ValueError-derived for argument errors."""
    if status == TTT_OK:
        return
    msg = ttt_status_string(status)
    if status == TTT_ERR_HIP:
        raise TTTError(status, msg)
    raise TTTArgumentError(status, msg)


def mode_bits(ln: str = "st", dual: bool = False, in_bf16: bool = False) -> int:
    m = 0
    if dual:
        m |= TTT_DUAL
    if in_bf16:
        m |= TTT_IN_BF16
    if ln == "exact":
        m |= TTT_LN_EXACT
    elif ln == "none":
        m |= TTT_NO_LN
    elif ln != "st":
        raise ValueError(f"unknown ln mode {ln!r}")
    return m


def forward(q, k, v, eta_logit, gate_logit, W0, gamma=None, beta=None, *, ln: str = "st",
            dual: bool = False, chunk: int = 16, out=None, W_final=None, stream=None):
    """Run the scan on torch device tensors; returns ``(out, W_final)``.

    q, k, v, gate_logit: [B,H,T,d] and eta_logit: [B,H,T], all float32 or all
    bfloat16; W0: [B,H,d,d] float32; gamma, beta: [H,d] float32 (not needed
    with ``ln="none"``).  ``out`` and ``W_final`` are allocated when not given
    (``W_final=W0`` updates the state in place).  Runs on ``stream`` (a
    ``torch.cuda.Stream``) or on the current stream.
    """
    import torch

    B, H, T, d = q.shape
    in_dtype = q.dtype
    if in_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"inputs must be float32 or bfloat16, got {in_dtype}")
    for name, t, shape in (("k", k, (B, H, T, d)), ("v", v, (B, H, T, d)),
                           ("gate_logit", gate_logit, (B, H, T, d)),
                           ("eta_logit", eta_logit, (B, H, T))):
        if t.dtype != in_dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {in_dtype}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if tuple(W0.shape) != (B, H, d, d) or W0.dtype != torch.float32:
        raise ValueError("W0 must be float32 [B,H,d,d]")
    if ln != "none":
        for name, t in (("gamma", gamma), ("beta", beta)):
            if t is None or tuple(t.shape) != (H, d) or t.dtype != torch.float32:
                raise ValueError(f"{name} must be float32 [H,d]")
    tensors = [q, k, v, eta_logit, gate_logit, W0] + ([gamma, beta] if ln != "none" else [])
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous device tensor")
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if W_final is None:
        W_final = torch.empty_like(W0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ptr = lambda t: None if t is None or t.numel() == 0 else t.data_ptr()
    status = ttt_linear_forward(
        ptr(q), ptr(k), ptr(v), ptr(eta_logit), ptr(gate_logit), W0.data_ptr(),
        ptr(gamma) if ln != "none" else None, ptr(beta) if ln != "none" else None,
        ptr(out), W_final.data_ptr(), B, H, T, d,
        mode_bits(ln, dual, in_dtype == torch.bfloat16), chunk if dual else 1,
        stream.cuda_stream)
    check(status)
    return out, W_final
