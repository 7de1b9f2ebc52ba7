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
TTT_SILU_QK = 16
TTT_FORCE_VALU = 32

#: bytes of the static device scratch behind ttt_linear_backward_noalloc
TTT_STATIC_SCRATCH_BYTES = 2097152

TTT_OK = 0
TTT_ERR_NULL = 1
TTT_ERR_SHAPE = 2
TTT_ERR_MODE = 3
TTT_ERR_UNSUPPORTED = 4
TTT_ERR_ALIAS = 5
TTT_ERR_HIP = 6
TTT_ERR_WORKSPACE = 7

# tokens per tile of the record; the dual form records only with chunks of this size
RECORD_CHUNK = 16

#: every symbol the header declares
EXPORTED = ("ttt_linear_backward", "ttt_linear_backward_kernel", "ttt_linear_backward_noalloc",
            "ttt_linear_backward_workspace_bytes",
            "ttt_linear_forward", "ttt_linear_forward_masked",
            "ttt_linear_forward_record", "ttt_linear_project",
            "ttt_linear_kernel", "ttt_linear_record_bytes", "ttt_linear_validate",
            "ttt_mlp_forward", "ttt_mlp_kernel", "ttt_mlp_validate",
            "ttt_status_string", "ttt_version")

_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ttt_linear call failed with status {status}: {message}")
        self.status = status


class TTTArgumentError(TTTError, ValueError):
    pass


def load_library(path: str = LIB_PATH, check_digest: bool = True) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built, or if
    it was built from other sources than the ones next to it (the digest that
    ``ttt_version()`` carries must match ``build.source_digest()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    # The library must share the HIP runtime of the framework that owns the
    # device memory: PyTorch ships its own libamdhip64, so it is loaded first
    # and the library's dependency then resolves to that copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.ttt_version.restype = ctypes.c_char_p
    lib.ttt_version.argtypes = []
    if check_digest:
        from .build import source_digest
        version = lib.ttt_version().decode()
        want = source_digest()
        if not version.endswith("src=" + want):
            raise RuntimeError(
                f"HIP library {path} is stale ({version!r}; the sources' digest is {want}): "
                "rebuild it (python -c 'import __graft_entry__ as g; g.build()')")
    lib.ttt_linear_forward.restype = ctypes.c_int32
    lib.ttt_linear_forward.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_linear_validate.restype = ctypes.c_int32
    lib.ttt_linear_validate.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_linear_kernel.restype = ctypes.c_char_p
    lib.ttt_linear_kernel.argtypes = [ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_linear_backward_kernel.restype = ctypes.c_char_p
    lib.ttt_linear_backward_kernel.argtypes = [ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_status_string.argtypes = [ctypes.c_int32]
    lib.ttt_mlp_forward.restype = ctypes.c_int32
    lib.ttt_mlp_forward.argtypes = [ctypes.c_void_p] * 12 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_mlp_validate.restype = ctypes.c_int32
    lib.ttt_mlp_validate.argtypes = [ctypes.c_void_p] * 12 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_mlp_kernel.restype = ctypes.c_char_p
    lib.ttt_mlp_kernel.argtypes = [ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64]
    lib.ttt_linear_forward_masked.restype = ctypes.c_int32
    lib.ttt_linear_forward_masked.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_linear_record_bytes.restype = ctypes.c_int32
    lib.ttt_linear_record_bytes.argtypes = [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.POINTER(ctypes.c_int64)]
    lib.ttt_linear_forward_record.restype = ctypes.c_int32
    lib.ttt_linear_forward_record.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int64] * 5 + [
        ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    lib.ttt_linear_backward.restype = ctypes.c_int32
    lib.ttt_linear_backward.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int64] +
                                        [ctypes.c_void_p] + [ctypes.c_int64] +
                                        [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 +
                                        [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p])
    lib.ttt_linear_backward_noalloc.restype = ctypes.c_int32
    lib.ttt_linear_backward_noalloc.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int64] +
                                                [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 +
                                                [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p])
    lib.ttt_linear_backward_workspace_bytes.restype = ctypes.c_int32
    lib.ttt_linear_backward_workspace_bytes.argtypes = [ctypes.c_int64] * 3 + [
        ctypes.c_uint32, ctypes.POINTER(ctypes.c_int64)]
    lib.ttt_linear_project.restype = ctypes.c_int32
    lib.ttt_linear_project.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64] * 5 + [
        ctypes.c_uint32, ctypes.c_void_p]
    _lib = lib
    return lib


def ttt_status_string(status: int) -> str:
    return load_library().ttt_status_string(int(status)).decode()


def ttt_linear_kernel(d: int, mode: int, chunk: int) -> str:
    """Name of the kernel family a valid call with these settings launches."""
    return load_library().ttt_linear_kernel(int(d), ctypes.c_uint32(int(mode)), int(chunk)).decode()


def ttt_linear_backward_kernel(d: int, mode: int, chunk: int) -> str:
    """Name of the kernel ttt_linear_backward runs with these settings."""
    return load_library().ttt_linear_backward_kernel(int(d), ctypes.c_uint32(int(mode)),
                                                     int(chunk)).decode()


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


def ttt_linear_forward_masked(q, k, v, eta_logit, gate_logit, W0, gamma, beta, update_mask,
                              out, W_final, B, H, T, d, mode, chunk, stream) -> int:
    """The dual-form scan with per-chunk SKIP/UPDATE decisions (raw pointers)."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_forward_masked(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W0), p(gamma), p(beta), p(update_mask),
        p(out), p(W_final), int(B), int(H), int(T), int(d), ctypes.c_uint32(int(mode)),
        int(chunk), p(stream)))


def ttt_linear_record_bytes(B, H, T, d, mode):
    """Returns ``(status, bytes)`` of the record a recording forward needs."""
    n = ctypes.c_int64(0)
    st = int(load_library().ttt_linear_record_bytes(int(B), int(H), int(T), int(d),
                                                    ctypes.c_uint32(int(mode)), ctypes.byref(n)))
    return st, int(n.value)


def ttt_linear_backward_workspace_bytes(B, H, d, mode):
    """Returns ``(status, bytes)`` of the workspace a backward call needs."""
    n = ctypes.c_int64(0)
    st = int(load_library().ttt_linear_backward_workspace_bytes(
        int(B), int(H), int(d), ctypes.c_uint32(int(mode)), ctypes.byref(n)))
    return st, int(n.value)


def ttt_linear_forward_record(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final,
                              record, record_bytes, B, H, T, d, mode, chunk, stream) -> int:
    """The recording forward with raw pointers; returns the status code."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_forward_record(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W0), p(gamma), p(beta), p(out),
        p(W_final), p(record), int(record_bytes), int(B), int(H), int(T), int(d),
        ctypes.c_uint32(int(mode)), int(chunk), p(stream)))


def ttt_linear_backward(q, k, v, eta_logit, gate_logit, gamma, beta, record, record_bytes,
                        workspace, workspace_bytes, dout, dW_final, dq, dk, dv, deta_logit,
                        dgate_logit, dW0, dgamma, dbeta, B, H, T, d, mode, chunk, stream) -> int:
    """The backward with raw pointers; returns the status code."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_backward(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(gamma), p(beta), p(record),
        int(record_bytes), p(workspace), int(workspace_bytes), p(dout), p(dW_final), p(dq),
        p(dk), p(dv), p(deta_logit),
        p(dgate_logit), p(dW0), p(dgamma), p(dbeta), int(B), int(H), int(T), int(d),
        ctypes.c_uint32(int(mode)), int(chunk), p(stream)))


def ttt_linear_backward_noalloc(q, k, v, eta_logit, gate_logit, gamma, beta, record,
                                record_bytes, dout, dW_final, dq, dk, dv, deta_logit,
                                dgate_logit, dW0, dgamma, dbeta, B, H, T, d, mode, chunk,
                                stream) -> int:
    """The backward with its scratch in the library's static device array
    (no workspace argument; raw pointers); returns the status code."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_linear_backward_noalloc(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(gamma), p(beta), p(record),
        int(record_bytes), p(dout), p(dW_final), p(dq), p(dk), p(dv), p(deta_logit),
        p(dgate_logit), p(dW0), p(dgamma), p(dbeta), int(B), int(H), int(T), int(d),
        ctypes.c_uint32(int(mode)), int(chunk), p(stream)))


def ttt_linear_project(x, w_proj, b_proj, q, k, v, eta_logit, gate_logit, B, T, hidden, H, d,
                       mode, stream) -> int:
    """The input projections with raw pointers; returns the status code."""
    lib = load_library()
    p = lambda x_: None if x_ is None else ctypes.c_void_p(int(x_))
    return int(lib.ttt_linear_project(
        p(x), p(w_proj), p(b_proj), p(q), p(k), p(v), p(eta_logit), p(gate_logit), int(B),
        int(T), int(hidden), int(H), int(d), ctypes.c_uint32(int(mode)), p(stream)))


def ttt_mlp_forward(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma, beta, out, W1_final,
                    W2_final, B, H, T, d, mode, chunk, stream) -> int:
    """The two-layer scan's C entry point with raw pointers (ints or None) and
    sizes; returns the status code unchanged."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_mlp_forward(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W1_0), p(W2_0), p(gamma), p(beta),
        p(out), p(W1_final), p(W2_final), int(B), int(H), int(T), int(d),
        ctypes.c_uint32(int(mode)), int(chunk), p(stream)))


def ttt_mlp_validate(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma, beta, out, W1_final,
                     W2_final, B, H, T, d, mode, chunk) -> int:
    """Only the argument checks of :func:`ttt_mlp_forward`; never launches."""
    lib = load_library()
    p = lambda x: None if x is None else ctypes.c_void_p(int(x))
    return int(lib.ttt_mlp_validate(
        p(q), p(k), p(v), p(eta_logit), p(gate_logit), p(W1_0), p(W2_0), p(gamma), p(beta),
        p(out), p(W1_final), p(W2_final), int(B), int(H), int(T), int(d),
        ctypes.c_uint32(int(mode)), int(chunk)))


def ttt_mlp_kernel(d: int, mode: int, chunk: int) -> str:
    """Name of the kernel a valid two-layer call with these settings launches."""
    return load_library().ttt_mlp_kernel(int(d), ctypes.c_uint32(int(mode)), int(chunk)).decode()


def check(status: int) -> None:
    """Raise for a non-OK status: ValueError-derived for argument errors."""
    if status == TTT_OK:
        return
    msg = ttt_status_string(status)
    if status == TTT_ERR_HIP:
        raise TTTError(status, msg)
    raise TTTArgumentError(status, msg)


def mode_bits(ln: str = "st", dual: bool = False, in_bf16: bool = False,
              silu_qk: bool = False, force_valu: bool = False) -> int:
    m = TTT_SILU_QK if silu_qk else 0
    if force_valu:
        m |= TTT_FORCE_VALU
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
            dual: bool = False, chunk: int = 16, out=None, W_final=None, stream=None,
            update_mask=None, silu_qk: bool = False, force_valu: bool = False):
    """Run the scan on torch device tensors; returns ``(out, W_final)``.

    q, k, v, gate_logit: [B,H,T,d] and eta_logit: [B,H,T], all float32 or all
    bfloat16; W0: [B,H,d,d] float32; gamma, beta: [H,d] float32 (not needed
    with ``ln="none"``).  ``out`` and ``W_final`` are allocated when not given
    (``W_final=W0`` updates the state in place).  Runs on ``stream`` (a
    ``torch.cuda.Stream``) or on the current stream.  ``update_mask`` (dual
    form only): uint8 [B,H,ceil(T/chunk)], 0 = SKIP the chunk's updates.
    ``silu_qk``: the :mlp variant (SiLU on q and k before the inner model).
    ``force_valu``: run the vector-ALU kernel even at d = 64.
    """
    import torch

    B, H, T, d = _check_inputs(q, k, v, eta_logit, gate_logit, W0, gamma, beta, ln)
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if W_final is None:
        W_final = torch.empty_like(W0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    mode = mode_bits(ln, dual, q.dtype == torch.bfloat16, silu_qk, force_valu)
    gb = (_ptr(gamma) if ln != "none" else None, _ptr(beta) if ln != "none" else None)
    if update_mask is not None:
        nc = -(-T // chunk) if T > 0 else 0
        if (update_mask.dtype != torch.uint8 or tuple(update_mask.shape) != (B, H, nc)
                or not update_mask.is_contiguous() or not update_mask.is_cuda):
            raise ValueError(f"update_mask must be a contiguous uint8 device tensor [B,H,{nc}]")
        status = ttt_linear_forward_masked(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta_logit), _ptr(gate_logit), W0.data_ptr(), *gb,
            _ptr(update_mask), _ptr(out), W_final.data_ptr(), B, H, T, d, mode, chunk,
            stream.cuda_stream)
    else:
        status = ttt_linear_forward(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta_logit), _ptr(gate_logit), W0.data_ptr(), *gb,
            _ptr(out), W_final.data_ptr(), B, H, T, d, mode, chunk if dual else 1,
            stream.cuda_stream)
    check(status)
    return out, W_final


def mlp_forward(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma=None, beta=None, *,
                ln: str = "st", dual: bool = False, chunk: int = 16, out=None, W1_final=None,
                W2_final=None, stream=None, force_valu: bool = False):
    """The scan with the two-layer inner model W2 silu(W1 x) on torch device
    tensors; returns ``(out, W1_final, W2_final)``.

    Inputs as in :func:`forward`, with W1_0 and W2_0 float32 [B,H,d,d] in
    place of W0.  Outputs are allocated when not given; ``W1_final=W1_0``
    (and likewise for W2) updates a state in place."""
    import torch

    B, H, T, d = _check_inputs(q, k, v, eta_logit, gate_logit, W1_0, gamma, beta, ln)
    if tuple(W2_0.shape) != (B, H, d, d) or W2_0.dtype != torch.float32 or not (
            W2_0.is_cuda and W2_0.is_contiguous()):
        raise ValueError("W2_0 must be a contiguous float32 device tensor [B,H,d,d]")
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if W1_final is None:
        W1_final = torch.empty_like(W1_0)
    if W2_final is None:
        W2_final = torch.empty_like(W2_0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    mode = mode_bits(ln, dual, q.dtype == torch.bfloat16, force_valu=force_valu)
    gb = (_ptr(gamma) if ln != "none" else None, _ptr(beta) if ln != "none" else None)
    status = ttt_mlp_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(eta_logit), _ptr(gate_logit), W1_0.data_ptr(),
        W2_0.data_ptr(), *gb, _ptr(out), W1_final.data_ptr(), W2_final.data_ptr(), B, H, T, d,
        mode, chunk if dual else 1, stream.cuda_stream)
    check(status)
    return out, W1_final, W2_final


def _ptr(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _check_inputs(q, k, v, eta_logit, gate_logit, W0, gamma, beta, ln):
    """Shape, dtype and placement checks shared by the tensor-level calls."""
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
    if W0 is not None and (tuple(W0.shape) != (B, H, d, d) or W0.dtype != torch.float32):
        raise ValueError("W0 must be float32 [B,H,d,d]")
    if ln != "none":
        for name, t in (("gamma", gamma), ("beta", beta)):
            if t is None or tuple(t.shape) != (H, d) or t.dtype != torch.float32:
                raise ValueError(f"{name} must be float32 [H,d]")
    tensors = [q, k, v, eta_logit, gate_logit] + ([] if W0 is None else [W0]) + (
        [gamma, beta] if ln != "none" else [])
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous device tensor")
    return B, H, T, d


def project(x, w_proj, b_proj=None, *, out_bf16: bool = True, stream=None):
    """The layer's input projections (:func:`ttt_linear_project`) on torch
    device tensors: x bfloat16 [B,T,hidden], w_proj bfloat16 [H,4d+1,hidden]
    (rows q, k, v, gate, eta per head), b_proj float32 [H,4d+1] or None.
    Returns ``(q, k, v, eta_logit, gate_logit)`` in the scan's layouts,
    bfloat16 (``out_bf16``) or float32, ready for :func:`forward`."""
    import torch

    if x.dim() != 3 or w_proj.dim() != 3 or x.shape[2] != w_proj.shape[2]:
        raise ValueError("x must be [B,T,hidden] and w_proj [H,4d+1,hidden]")
    if x.dtype != torch.bfloat16 or w_proj.dtype != torch.bfloat16:
        raise ValueError("x and w_proj must be bfloat16")
    B, T, hidden = x.shape
    H, rows, _ = w_proj.shape
    d = (rows - 1) // 4
    if rows != 4 * d + 1:
        raise ValueError("w_proj must have 4d+1 rows per head")
    if b_proj is not None and (b_proj.dtype != torch.float32 or tuple(b_proj.shape) != (H, rows)):
        raise ValueError("b_proj must be float32 [H,4d+1]")
    for t in (x, w_proj) + (() if b_proj is None else (b_proj,)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous device tensor")
    dt = torch.bfloat16 if out_bf16 else torch.float32
    opt = dict(dtype=dt, device=x.device)
    q, k, v, gate = (torch.empty((B, H, T, d), **opt) for _ in range(4))
    eta = torch.empty((B, H, T), **opt)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    mode = TTT_IN_BF16 if out_bf16 else 0
    check(ttt_linear_project(x.data_ptr(), w_proj.data_ptr(),
                             None if b_proj is None else b_proj.data_ptr(), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(eta), _ptr(gate), B, T, hidden, H, d, mode,
                             stream.cuda_stream))
    return q, k, v, eta, gate


def forward_record(q, k, v, eta_logit, gate_logit, W0, gamma=None, beta=None, *,
                   ln: str = "st", out=None, W_final=None, record=None, stream=None,
                   silu_qk: bool = False, dual: bool = False, chunk: int = RECORD_CHUNK,
                   force_valu: bool = False):
    """:func:`forward` that also returns the record the backward reads:
    ``(out, W_final, record)``, the record a uint8 device tensor.  Every d and
    mode of :func:`forward` (``chunk`` is the dual form's)."""
    import torch

    B, H, T, d = _check_inputs(q, k, v, eta_logit, gate_logit, W0, gamma, beta, ln)
    mode = mode_bits(ln, dual, q.dtype == torch.bfloat16, silu_qk, force_valu)
    st, nbytes = ttt_linear_record_bytes(B, H, T, d, mode)
    check(st)
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if W_final is None:
        W_final = torch.empty_like(W0)
    if record is None:
        record = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    check(ttt_linear_forward_record(
        _ptr(q), _ptr(k), _ptr(v), _ptr(eta_logit), _ptr(gate_logit), W0.data_ptr(),
        _ptr(gamma) if ln != "none" else None, _ptr(beta) if ln != "none" else None,
        _ptr(out), W_final.data_ptr(), record.data_ptr(), record.numel() * record.element_size(),
        B, H, T, d, mode, chunk if dual else 1, stream.cuda_stream))
    return out, W_final, record


def backward(q, k, v, eta_logit, gate_logit, gamma, beta, record, dout, dW_final=None, *,
             ln: str = "st", stream=None, silu_qk: bool = False, dual: bool = False,
             chunk: int = RECORD_CHUNK, workspace=None, force_valu: bool = False):
    """Gradients from a record of :func:`forward_record` (same ``ln``,
    ``silu_qk``, ``dual`` and ``chunk``; ``force_valu`` runs the vector-ALU
    backward where the matrix-core one applies) and dL/dout (float32 [B,H,T,d]), dL/dW_final
    (float32 [B,H,d,d] or None).  Returns a dict with dq, dk, dv, dgate_logit,
    deta_logit, dW0, dgamma, dbeta (float32; the last two None with
    ``ln="none"``).  ``workspace``: a uint8 device tensor of at least
    ``ttt_linear_backward_workspace_bytes`` bytes (allocated when None)."""
    import torch

    B, H, T, d = _check_inputs(q, k, v, eta_logit, gate_logit, None, gamma, beta, ln)
    if dout.dtype != torch.float32 or tuple(dout.shape) != (B, H, T, d) or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous float32 [B,H,T,d] tensor")
    if dW_final is not None and (dW_final.dtype != torch.float32 or not dW_final.is_contiguous()
                                 or tuple(dW_final.shape) != (B, H, d, d)):
        raise ValueError("dW_final must be a contiguous float32 [B,H,d,d] tensor")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dq=torch.empty((B, H, T, d), **f32), dk=torch.empty((B, H, T, d), **f32),
             dv=torch.empty((B, H, T, d), **f32), dgate_logit=torch.empty((B, H, T, d), **f32),
             deta_logit=torch.empty((B, H, T), **f32), dW0=torch.empty((B, H, d, d), **f32),
             dgamma=None if ln == "none" else torch.empty((H, d), **f32),
             dbeta=None if ln == "none" else torch.empty((H, d), **f32))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    mode = mode_bits(ln, dual, q.dtype == torch.bfloat16, silu_qk, force_valu)
    st, ws_bytes = ttt_linear_backward_workspace_bytes(B, H, d, mode)
    check(st)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    check(ttt_linear_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(eta_logit), _ptr(gate_logit),
        _ptr(gamma) if ln != "none" else None, _ptr(beta) if ln != "none" else None,
        record.data_ptr(), record.numel() * record.element_size(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(dout),
        None if dW_final is None else dW_final.data_ptr(), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["deta_logit"]), _ptr(g["dgate_logit"]), g["dW0"].data_ptr(),
        _ptr(g["dgamma"]), _ptr(g["dbeta"]), B, H, T, d, mode, chunk if dual else 1,
        stream.cuda_stream))
    return g


_autograd_fn = None


def ttt_linear(q, k, v, eta_logit, gate_logit, W0, gamma=None, beta=None, *, ln: str = "st",
               silu_qk: bool = False, dual: bool = False, chunk: int = RECORD_CHUNK):
    """Differentiable scan for torch autograd: ``(out, W_final)``.

    The forward is :func:`forward_record`; the backward is :func:`backward`
    on the saved record.  Every d and mode of :func:`forward`.  Gradients come
    back in float32 (autograd casts them to a bf16 input's dtype).
    """
    global _autograd_fn
    if _autograd_fn is None:
        import torch

        class TTTLinearFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, eta_logit, gate_logit, W0, gamma, beta, ln, silu_qk, dual,
                        chunk):
                out, W_final, record = forward_record(q, k, v, eta_logit, gate_logit, W0, gamma,
                                                      beta, ln=ln, silu_qk=silu_qk, dual=dual,
                                                      chunk=chunk)
                ctx.ln = ln
                ctx.silu_qk = silu_qk
                ctx.dual = dual
                ctx.chunk = chunk
                ctx.save_for_backward(q, k, v, eta_logit, gate_logit, gamma, beta, record)
                return out, W_final

            @staticmethod
            def backward(ctx, dout, dW_final):
                q, k, v, eta_logit, gate_logit, gamma, beta, record = ctx.saved_tensors
                B, H, T, d = q.shape
                if dout is None:
                    dout = torch.zeros((B, H, T, d), dtype=torch.float32, device=q.device)
                g = backward(q, k, v, eta_logit, gate_logit, gamma, beta, record,
                             dout.contiguous().float(),
                             None if dW_final is None else dW_final.contiguous().float(),
                             ln=ctx.ln, silu_qk=ctx.silu_qk, dual=ctx.dual, chunk=ctx.chunk)
                return (g["dq"], g["dk"], g["dv"], g["deta_logit"], g["dgate_logit"], g["dW0"],
                        g["dgamma"], g["dbeta"], None, None, None, None)

        _autograd_fn = TTTLinearFunction
    if ln == "none":
        gamma = beta = None
    return _autograd_fn.apply(q, k, v, eta_logit, gate_logit, W0, gamma, beta, ln, silu_qk, dual,
                              chunk)
