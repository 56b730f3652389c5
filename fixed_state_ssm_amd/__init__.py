"""Interdomain Attention token mixer on AMD MI355X (gfx950).

The work runs in libidattn.so (HIP kernels behind a C ABI, include/idattn.h).
This package holds the ctypes binding (functions named like the C entry
points) and conveniences, forward(), forward_normalized(), forward_varlen()
(and forward_varlen_into() for caller-provided outputs), decode_step() and
backward(), that allocate outputs and workspace with PyTorch and call the
binding on the current stream.
"""
from __future__ import annotations

from .binding import (ALGO, EXPORTS, IdattnParamGrads, idattn_backward, idattn_backward_workspace_size,
                      make_param_grads, FEATURE_NORM, IO, LIB_PATH, STATUS, IdattnDims, IdattnError, IdattnParams,
                      NOALLOC_SCRATCH_BYTES, idattn_decode_step, idattn_decode_step_normalized, idattn_forward,
                      idattn_forward_noalloc,
                      idattn_forward_normalized,
                      idattn_forward_normalized_workspace_size, idattn_forward_varlen,
                      idattn_forward_varlen_workspace_size, idattn_forward_workspace_size,
                      idattn_last_error, idattn_status_string, idattn_version, load_library,
                      make_dims, make_params)

__all__ = ["IdattnParamGrads", "idattn_backward", "idattn_backward_workspace_size", "make_param_grads", "backward",
           "ALGO", "EXPORTS", "NOALLOC_SCRATCH_BYTES", "idattn_forward_noalloc", "FEATURE_NORM", "IO", "LIB_PATH", "STATUS", "IdattnDims", "IdattnError", "IdattnParams",
           "idattn_decode_step", "idattn_decode_step_normalized", "idattn_forward", "idattn_forward_normalized",
           "idattn_forward_normalized_workspace_size", "idattn_forward_varlen", "idattn_forward_varlen_workspace_size",
           "idattn_forward_workspace_size",
           "idattn_last_error", "idattn_status_string", "idattn_version", "load_library",
           "make_dims", "make_params", "forward", "forward_normalized", "forward_varlen", "forward_varlen_into",
           "decode_step",
           "params_to_device"]

PARAM_KEYS = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc")


def params_to_device(p: dict, device="cuda"):
    """Copy a dict of float32 arrays/tensors (the idattn_params layout, with
    rff_omega when present) to the device."""
    import torch
    keys = PARAM_KEYS + (("rff_omega",) if p.get("rff_omega") is not None else ())
    return {k: torch.as_tensor(p[k], dtype=torch.float32).contiguous().to(device) for k in keys}


def _io_name(t):
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t.dtype}")


def forward(q, k, v, params: dict, *, state_in=None, tail_in=None, return_state=False,
            algo="auto", eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared", stream=None):
    """o = mixer(q, k, v) for q, k, v of shape [B, N, H, d] on the GPU.

    params: device tensors (see params_to_device).  state_in: float32
    [B, H, M, 2d, 2] or None; tail_in: [B, H, 2, W-1, d] in q's dtype or None.
    With return_state=True returns (o, state_out, tail_out)."""
    import torch
    B, N, H, d = q.shape
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    io = _io_name(q)
    for t in (k, v):
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k, v must share shape and dtype")
    dims = make_dims(B, N, H, d, M, W, io, algo, eps_feat, eps_norm, feature_norm)
    nbytes = idattn_forward_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    state_out = tail_out = None
    if return_state:
        state_out = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device=q.device)
        tail_out = torch.empty((B, H, 2, W - 1, d), dtype=q.dtype, device=q.device)
    idattn_forward(dims, make_params(params), q, k, v, o, state_in, tail_in, state_out, tail_out,
                   ws, nbytes, stream)
    return (o, state_out, tail_out) if return_state else o


def forward_normalized(q, k, v, params: dict, *, state_in=None, tail_in=None, eta_in=None, return_state=False,
                       algo="auto", eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared", stream=None):
    """o = mixer with the normalised readout (eta state) for q, k, v
    [B, N, H, d].  eta_in: float32 [B, H, M, 2] or None.  With
    return_state=True returns (o, state_out, tail_out, eta_out)."""
    import torch
    B, N, H, d = q.shape
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    for t in (k, v):
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k, v must share shape and dtype")
    dims = make_dims(B, N, H, d, M, W, _io_name(q), algo, eps_feat, eps_norm, feature_norm)
    nbytes = idattn_forward_normalized_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    state_out = tail_out = eta_out = None
    if return_state:
        state_out = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device=q.device)
        tail_out = torch.empty((B, H, 2, W - 1, d), dtype=q.dtype, device=q.device)
        eta_out = torch.empty((B, H, M, 2), dtype=torch.float32, device=q.device)
    idattn_forward_normalized(dims, make_params(params), q, k, v, o, state_in, tail_in, eta_in, state_out, tail_out,
                              eta_out, ws, nbytes, stream)
    return (o, state_out, tail_out, eta_out) if return_state else o


def forward_varlen(q, k, v, params: dict, cu_seqlens, *, state_in=None, tail_in=None, return_state=False,
                   algo="auto", eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared", stream=None,
                   host_lengths=False):
    """o = mixer over a packed batch: q, k, v [T, H, d] on the GPU hold B
    sequences end to end, sequence b being tokens cu_seqlens[b] ..
    cu_seqlens[b+1]-1 (cu_seqlens: int32 device tensor [B + 1]).  state_in
    [B, H, M, 2d, 2] and tail_in [B, H, 2, W-1, d] or None.  host_lengths
    also hands a host copy of the table to the library, which checks it (one
    device-to-host copy).  With return_state=True returns (o, state_out,
    tail_out)."""
    import torch
    T, H, d = q.shape
    B = cu_seqlens.shape[0] - 1
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    state_out = tail_out = None
    if return_state:
        state_out = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device=q.device)
        tail_out = torch.empty((B, H, 2, W - 1, d), dtype=q.dtype, device=q.device)
    o = forward_varlen_into(q, k, v, params, cu_seqlens, state_in=state_in, tail_in=tail_in, state_out=state_out,
                            tail_out=tail_out, algo=algo, eps_feat=eps_feat, eps_norm=eps_norm,
                            feature_norm=feature_norm, stream=stream, host_lengths=host_lengths)
    return (o, state_out, tail_out) if return_state else o


def forward_varlen_into(q, k, v, params: dict, cu_seqlens, *, o=None, state_in=None, tail_in=None, state_out=None,
                        tail_out=None, algo="auto", eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared",
                        stream=None, host_lengths=False):
    """forward_varlen into caller-provided outputs (any of o, state_out,
    tail_out; o is allocated when None): state_out may be state_in and
    tail_out tail_in (in place).  Returns o."""
    import torch
    T, H, d = q.shape
    B = cu_seqlens.shape[0] - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    for t in (k, v):
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k, v must share shape and dtype")
    dims = make_dims(B, T, H, d, M, W, _io_name(q), algo, eps_feat, eps_norm, feature_norm)
    nbytes = idattn_forward_varlen_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    host = cu_seqlens.cpu().tolist() if host_lengths else None
    idattn_forward_varlen(dims, make_params(params), cu_seqlens, q, k, v, o, state_in, tail_in, state_out, tail_out,
                          ws, nbytes, stream, cu_seqlens_host=host)
    return o


def backward(q, k, v, params: dict, grad_o, *, state_in=None, tail_in=None, grad_state=None, eps_feat=1e-6,
             eps_norm=1e-6, feature_norm="squared", stream=None):
    """Gradients of sum(grad_o * o) + Re sum(conj(grad_state) * state_out) for
    the forward over q, k, v [B, N, H, d] (same dtype for all) with params,
    state_in and tail_in.  Returns a dict: q, k, v (q's dtype), the parameter
    keys (float32, shaped like the parameters) and state (float32 [B, H, M,
    2d, 2], the state_in gradient)."""
    import torch
    B, N, H, d = q.shape
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    dims = make_dims(B, N, H, d, M, W, _io_name(q), "auto", eps_feat, eps_norm, feature_norm)
    nbytes = idattn_backward_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    out = {"q": torch.empty_like(q), "k": torch.empty_like(k), "v": torch.empty_like(v)}
    for key in PARAM_KEYS:
        out[key] = torch.empty_like(params[key])
    out["state"] = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device=q.device)
    idattn_backward(dims, make_params(params), q, k, v, state_in, tail_in, grad_o, grad_state, out["q"], out["k"],
                    out["v"], make_param_grads(out), out["state"], ws, nbytes, stream)
    return out


def decode_step(q_t, k_t, v_t, params: dict, state, tail, *, eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared",
                eta=None, stream=None):
    """One token per sequence, q_t, k_t, v_t [B, H, d], or 1..8 tokens,
    [B, N, H, d]; state float32 [B, H, M, 2d, 2] and tail [B, H, 2, W-1, d]
    are updated in place.  With eta (float32 [B, H, M, 2], updated in place)
    the readout is the normalised one.  Returns o_t shaped like q_t."""
    import torch
    if q_t.dim() == 3:
        B, H, d = q_t.shape
        N = 1
    else:
        B, N, H, d = q_t.shape
    M = params["A"].shape[1]
    W = params["conv_q"].shape[-1]
    dims = make_dims(B, N, H, d, M, W, _io_name(q_t), "auto", eps_feat, eps_norm, feature_norm)
    o_t = torch.empty_like(q_t)
    if eta is None:
        idattn_decode_step(dims, make_params(params), q_t, k_t, v_t, o_t, state, tail, stream)
    else:
        idattn_decode_step_normalized(dims, make_params(params), q_t, k_t, v_t, o_t, state, tail, eta, stream)
    return o_t
