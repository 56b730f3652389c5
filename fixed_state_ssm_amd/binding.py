"""ctypes binding of libidattn.so (argument marshalling only).

Every function named idattn_* here calls the C entry point of the same name
in include/idattn.h; the arithmetic of the mixer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libidattn.so")

STATUS = {0: "IDATTN_OK", 1: "IDATTN_ERR_NULL", 2: "IDATTN_ERR_SHAPE", 3: "IDATTN_ERR_UNSUPPORTED",
          4: "IDATTN_ERR_WORKSPACE", 5: "IDATTN_ERR_ALIAS", 6: "IDATTN_ERR_ARG", 7: "IDATTN_ERR_HIP"}
IO = {"f32": 0, "bf16": 1}
ALGO = {"auto": 0, "sequential": 1, "chunked": 2}
FEATURE_NORM = {"squared": 0, "unit": 1, "rff": 2}

EXPORTS = ("idattn_forward_workspace_size", "idattn_forward", "idattn_forward_noalloc",
           "idattn_forward_normalized_workspace_size",
           "idattn_forward_normalized", "idattn_forward_varlen_workspace_size", "idattn_forward_varlen",
           "idattn_decode_step", "idattn_decode_step_normalized", "idattn_backward_workspace_size",
           "idattn_backward", "idattn_status_string", "idattn_last_error", "idattn_version")


class IdattnDims(ctypes.Structure):
    _fields_ = [("B", c_int64), ("N", c_int64), ("H", c_int64), ("d", c_int64), ("M", c_int64),
                ("W", c_int64), ("io_dtype", c_int32), ("algo", c_int32),
                ("eps_feat", c_float), ("eps_norm", c_float), ("feature_norm", c_int32)]


class IdattnParams(ctypes.Structure):
    _fields_ = [("conv_q", c_void_p), ("conv_k", c_void_p), ("gain", c_void_p), ("bias", c_void_p),
                ("log_dt", c_void_p), ("A", c_void_p), ("Bc", c_void_p), ("rff_omega", c_void_p)]


class IdattnParamGrads(ctypes.Structure):
    _fields_ = [("conv_q", c_void_p), ("conv_k", c_void_p), ("gain", c_void_p), ("bias", c_void_p),
                ("log_dt", c_void_p), ("A", c_void_p), ("Bc", c_void_p)]


class IdattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libidattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fixed_state_ssm_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.idattn_forward_workspace_size.argtypes = [P(IdattnDims), P(c_size_t)]
    lib.idattn_forward_workspace_size.restype = c_int
    lib.idattn_forward.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 9 + [c_size_t, c_void_p]
    lib.idattn_forward.restype = c_int
    lib.idattn_forward_noalloc.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 9
    lib.idattn_forward_noalloc.restype = c_int
    lib.idattn_forward_normalized_workspace_size.argtypes = [P(IdattnDims), P(c_size_t)]
    lib.idattn_forward_normalized_workspace_size.restype = c_int
    lib.idattn_forward_normalized.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 11 + [c_size_t, c_void_p]
    lib.idattn_forward_normalized.restype = c_int
    lib.idattn_forward_varlen_workspace_size.argtypes = [P(IdattnDims), P(c_size_t)]
    lib.idattn_forward_varlen_workspace_size.restype = c_int
    lib.idattn_forward_varlen.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 11 + [c_size_t, c_void_p]
    lib.idattn_forward_varlen.restype = c_int
    lib.idattn_decode_step_normalized.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 8
    lib.idattn_decode_step_normalized.restype = c_int
    lib.idattn_decode_step.argtypes = [P(IdattnDims), P(IdattnParams)] + [c_void_p] * 7
    lib.idattn_decode_step.restype = c_int
    lib.idattn_backward_workspace_size.argtypes = [P(IdattnDims), P(c_size_t)]
    lib.idattn_backward_workspace_size.restype = c_int
    lib.idattn_backward.argtypes = ([P(IdattnDims), P(IdattnParams)] + [c_void_p] * 10 + [P(IdattnParamGrads)]
                                    + [c_void_p, c_void_p, c_size_t, c_void_p])
    lib.idattn_backward.restype = c_int
    lib.idattn_status_string.argtypes = [c_int]
    lib.idattn_status_string.restype = ctypes.c_char_p
    lib.idattn_last_error.argtypes = []
    lib.idattn_last_error.restype = ctypes.c_char_p
    lib.idattn_version.argtypes = []
    lib.idattn_version.restype = c_int
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling
def _ptr(x):
    """None -> NULL; int -> that address; torch tensor -> its data pointer
    (must be contiguous)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return x.data_ptr() or None
    raise TypeError(f"cannot pass {type(x).__name__} as a pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _check(status: int):
    if status != 0:
        detail = load_library().idattn_last_error().decode(errors="replace")
        raise IdattnError(status, detail)


def make_dims(B, N, H, d, M, W=4, io="bf16", algo="auto", eps_feat=1e-6, eps_norm=1e-6,
              feature_norm="squared") -> IdattnDims:
    return IdattnDims(int(B), int(N), int(H), int(d), int(M), int(W), IO[io] if isinstance(io, str) else int(io),
                      ALGO[algo] if isinstance(algo, str) else int(algo), float(eps_feat), float(eps_norm),
                      FEATURE_NORM[feature_norm] if isinstance(feature_norm, str) else int(feature_norm))


def make_params(p: dict) -> IdattnParams:
    """p: dict of float32 device tensors conv_q, conv_k, gain, bias, log_dt, A, Bc
    and, for the RFF feature map, rff_omega [H, d, d/2] (else absent or None).
    The caller keeps the tensors alive while the struct is in use."""
    keys = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc")
    return IdattnParams(*(_ptr(p[k]) for k in keys), _ptr(p.get("rff_omega")))


# ------------------------------------------------------------------ C entry points
def idattn_version() -> int:
    return load_library().idattn_version()


def idattn_status_string(status: int) -> str:
    return load_library().idattn_status_string(int(status)).decode()


def idattn_last_error() -> str:
    return load_library().idattn_last_error().decode(errors="replace")


def idattn_forward_workspace_size(dims: IdattnDims) -> int:
    out = c_size_t(0)
    _check(load_library().idattn_forward_workspace_size(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def idattn_forward(dims, params, q, k, v, o, state_in=None, tail_in=None, state_out=None,
                   tail_out=None, workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load_library().idattn_forward(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
        _ptr(state_in), _ptr(tail_in), _ptr(state_out), _ptr(tail_out), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def idattn_forward_noalloc(dims, params, q, k, v, o, state_in=None, tail_in=None, state_out=None,
                           tail_out=None, stream=None) -> None:
    _check(load_library().idattn_forward_noalloc(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
        _ptr(state_in), _ptr(tail_in), _ptr(state_out), _ptr(tail_out), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 192 << 20


def idattn_forward_normalized_workspace_size(dims: IdattnDims) -> int:
    out = c_size_t(0)
    _check(load_library().idattn_forward_normalized_workspace_size(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def idattn_forward_normalized(dims, params, q, k, v, o, state_in=None, tail_in=None, eta_in=None, state_out=None,
                              tail_out=None, eta_out=None, workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load_library().idattn_forward_normalized(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state_in),
        _ptr(tail_in), _ptr(eta_in), _ptr(state_out), _ptr(tail_out), _ptr(eta_out), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def idattn_forward_varlen_workspace_size(dims: IdattnDims) -> int:
    out = c_size_t(0)
    _check(load_library().idattn_forward_varlen_workspace_size(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def idattn_forward_varlen(dims, params, cu_seqlens, q, k, v, o, state_in=None, tail_in=None, state_out=None,
                          tail_out=None, workspace=None, workspace_bytes=0, stream=None, cu_seqlens_host=None) -> None:
    """cu_seqlens: device int32 table (tensor or address); cu_seqlens_host:
    None or a host copy (sequence of ints), which the library checks."""
    host = None
    if cu_seqlens_host is not None:
        vals = [int(x) for x in cu_seqlens_host]
        host = (ctypes.c_int32 * len(vals))(*vals)
    _check(load_library().idattn_forward_varlen(
        ctypes.byref(dims), ctypes.byref(params), _ptr(cu_seqlens), host, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
        _ptr(state_in), _ptr(tail_in), _ptr(state_out), _ptr(tail_out), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def make_param_grads(g: dict) -> IdattnParamGrads:
    """g: dict of float32 device tensors conv_q, conv_k, gain, bias, log_dt,
    A, Bc shaped like the parameters (the outputs of idattn_backward)."""
    keys = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc")
    return IdattnParamGrads(*(_ptr(g[k]) for k in keys))


def idattn_backward_workspace_size(dims: IdattnDims) -> int:
    out = c_size_t(0)
    _check(load_library().idattn_backward_workspace_size(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def idattn_backward(dims, params, q, k, v, state_in, tail_in, grad_o, grad_state, grad_q, grad_k, grad_v,
                    grad_params, grad_state_in=None, workspace=None, workspace_bytes=0, stream=None) -> None:
    _check(load_library().idattn_backward(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(tail_in),
        _ptr(grad_o), _ptr(grad_state), _ptr(grad_q), _ptr(grad_k), _ptr(grad_v), ctypes.byref(grad_params),
        _ptr(grad_state_in), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def idattn_decode_step(dims, params, q_t, k_t, v_t, o_t, state, tail, stream=None) -> None:
    _check(load_library().idattn_decode_step(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(o_t),
        _ptr(state), _ptr(tail), _stream(stream)))


def idattn_decode_step_normalized(dims, params, q_t, k_t, v_t, o_t, state, tail, eta, stream=None) -> None:
    _check(load_library().idattn_decode_step_normalized(
        ctypes.byref(dims), ctypes.byref(params), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(o_t),
        _ptr(state), _ptr(tail), _ptr(eta), _stream(stream)))
