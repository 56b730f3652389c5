"""fp64 backward of the Interdomain Attention token mixer (gradients of a
scalar loss with respect to the inputs, the parameters and the carried state).

TEST INFRASTRUCTURE, like the rest of this package.  The forward pass is
written out again, literally and in the same order as idattn_oracle.forward,
with PyTorch CPU tensors in float64 / complex128, so that torch.autograd
differentiates it; nothing here is blocked, fused or reordered.  The pages
train the layer inside language models (Chinese rendering, section 1; German
summary, "Skalierbare Implementierung"), which needs these gradients; they
print no backward pass, so the gradients are those of the forward exactly as
the oracle reads it (the readings listed in idattn_oracle's header apply).

Pins (tests/oracle_pins.py):
  forward_torch  pinned: equals idattn_oracle.forward (NumPy) on the same
                 inputs, for every feature map.
  backward       pinned: directional derivatives against central finite
                 differences of idattn_oracle.forward (NumPy, not this file),
                 for q, k, v, every parameter and the carried state.
"""
from __future__ import annotations

import numpy as np
import torch

F64 = torch.float64
C128 = torch.complex128

PARAM_KEYS = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc")


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def forward_torch(q, k, v, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None,
                  feature_norm="squared"):
    """The forward of idattn_oracle.forward in torch float64 (differentiable).

    q, k, v [B, N, H, d]; params: tensors conv_q, conv_k [H, d, W], gain, bias
    [H, 2d], log_dt [H], A, Bc [H, M, 2] (and rff_omega [H, d, d/2] for the
    RFF map); state_in complex [B, H, M, 2d] or None; tail_in [B, H, 2, W-1, d]
    or None.  Returns (o [B, N, H, d], state_out complex [B, H, M, 2d])."""
    B, N, H, d = q.shape
    W = params["conv_q"].shape[-1]
    M = params["A"].shape[1]
    if tail_in is None:
        tail_in = torch.zeros((B, H, 2, W - 1, d), dtype=F64)
    if state_in is None:
        state_in = torch.zeros((B, H, M, 2 * d), dtype=C128)

    def conv(x, w, hist):
        # c(i) = sum_j w[..., j] x(i - W + 1 + j), history before position 0 from hist
        xp = torch.cat([hist.permute(0, 2, 1, 3), x], dim=1)
        c = torch.zeros_like(x)
        for j in range(W):
            c = c + xp[:, j:j + N] * w[None, None, :, :, j]
        return c

    c_q = conv(q, params["conv_q"], tail_in[:, :, 0])
    c_k = conv(k, params["conv_k"], tail_in[:, :, 1])
    if feature_norm == "rff":
        om = params["rff_omega"]
        D = om.shape[-1]

        def fmap(c):
            ph = torch.einsum("bnhi,hif->bnhf", c, om)
            return torch.cat([torch.cos(ph), torch.sin(ph)], dim=-1) / np.sqrt(D)
    else:
        def fmap(c):
            y = c * torch.sigmoid(c)
            n2 = (y * y).sum(-1, keepdim=True) + eps_feat
            return y / (n2 if feature_norm == "squared" else torch.sqrt(n2))
    xi_q, xi_k = fmap(c_q), fmap(c_k)

    def rms(x, g, b):
        return g[None, None] * x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps_norm) + b[None, None]

    z_k = rms(xi_k, params["gain"][:, :d], params["bias"][:, :d])
    z_v = rms(v, params["gain"][:, d:], params["bias"][:, d:])

    dt = torch.exp(params["log_dt"])[:, None]
    lam = torch.complex(params["A"][..., 0], params["A"][..., 1])
    bc = torch.complex(params["Bc"][..., 0], params["Bc"][..., 1])
    abar = torch.exp(dt * lam)
    bbar = (abar - 1.0) / lam * bc  # lambda != 0 here (Re lambda < 0)
    a4, b4 = abar[None, :, :, None], bbar[None, :, :, None]

    U = state_in[..., :d]
    G = state_in[..., d:]
    outs = []
    for i in range(N):
        U = a4 * U + b4 * z_k[:, i, :, None, :].to(C128)
        G = a4 * G + b4 * z_v[:, i, :, None, :].to(C128)
        s = torch.einsum("bhr,bhmr->bhm", xi_q[:, i].to(C128), U)
        outs.append(torch.einsum("bhm,bhmc->bhc", s, G).real)
    o = torch.stack(outs, dim=1)
    return o, torch.cat([U, G], dim=-1)


def backward(q, k, v, params, grad_o, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None,
             grad_state=None, feature_norm="squared"):
    """Gradients of L = sum(grad_o * o) + Re sum(conj(grad_state) * state_out)
    (grad_state complex [B, H, M, 2d] or None) with respect to q, k, v, each
    parameter of PARAM_KEYS and, when given, state_in (as d/dRe + i d/dIm).
    Inputs are NumPy arrays; returns a dict of NumPy arrays shaped like them."""
    leaves = {"q": _t(q), "k": _t(k), "v": _t(v)}
    for key in PARAM_KEYS:
        leaves[key] = _t(params[key])
    p = {key: leaves[key] for key in PARAM_KEYS}
    if feature_norm == "rff":
        p["rff_omega"] = _t(params["rff_omega"])
    st = None
    if state_in is not None:
        z = np.asarray(state_in, dtype=np.complex128)
        leaves["state_re"], leaves["state_im"] = _t(z.real), _t(z.imag)
    for t in leaves.values():
        t.requires_grad_(True)
    if state_in is not None:
        st = torch.complex(leaves["state_re"], leaves["state_im"])
    tl = None if tail_in is None else _t(tail_in)
    o, st_out = forward_torch(leaves["q"], leaves["k"], leaves["v"], p, eps_feat, eps_norm, st, tl, feature_norm)
    loss = (o * _t(grad_o)).sum()
    if grad_state is not None:
        gs = torch.as_tensor(np.asarray(grad_state, dtype=np.complex128))
        loss = loss + (st_out * gs.conj()).real.sum()
    names = list(leaves)
    grads = torch.autograd.grad(loss, [leaves[n] for n in names], allow_unused=True)
    out = {}
    for n, g in zip(names, grads):
        out[n] = np.zeros(leaves[n].shape) if g is None else g.detach().numpy()
    if state_in is not None:
        out["state"] = out.pop("state_re") + 1j * out.pop("state_im")
    return out
