"""Literal fp64 oracle of the Interdomain Attention token-mixer forward pass.

TEST INFRASTRUCTURE.  Plain NumPy, float64 / complex128, a Python loop over
time with each step vectorised over (batch, head, mode, channel).  Slow and
meant to be read against the pages by eye.

Pages cited (all about arXiv 2605.24330, "Interdomain Attention: Beyond
Token-Level Key-Value Memory"):
  p1  "Interdomain Attention: 超越令牌级键值记忆" - Chinese rendering of the
      arXiv HTML (bittide.aicompass.dev).  Sections 2 (attention as kernel
      regression, eq. 1; SSMs and HiPPO), 3 (Fig. 1), 3.1 (eqs. 3-6).
  p2  gist.science German summary, "Technische Zusammenfassung":
      "Theoretische Herleitung" and "Skalierbare Implementierung".
  p3  gist.science Dutch summary, "Technische Samenvatting":
      "Schaalbare Implementatie" (same content as p2).

What the scalable layer computes, per batch row b, head h and position i
(p2 "Skalierbare Implementierung", all four bullets; p3 the same bullets):
  1. c = SC(x): causal depthwise short convolution of q and of k.
  2. xi = SiLU(c) / ||SiLU(c)||^2 over the R = d channels of the head.
  3. z_k = RMSNorm(xi_k) and z_v = RMSNorm(v), each half with its own
     per-head gain and bias, before the SSM.
  4. One complex-diagonal S4D system per head, ZOH-discretised:
     abar = exp(Delta*lambda), bbar = (abar - 1)/lambda * B.
  5. Driven by the concatenation [z_k, z_v]:
     U_m(i) = abar_m U_m(i-1) + bbar_m z_k(i)          (M x R)
     Gamma_m(i) = abar_m Gamma_m(i-1) + bbar_m z_v(i)  (M x d)
  6. Mode scores s_m(i) = xi_q(i) . U_m(i)  (F_q U^T, N_q x M; p1 Fig. 1).
  7. Denominator-free readout o_i = Re sum_m s_m(i) Gamma_m(i)
     (F_q U^T Gamma; p2 last implementation bullet; eta is dropped).

Readings where the pages are silent (each also listed in the design notes):
  - the norm in xi is squared as printed on p2/p3, with eps_feat added;
  - RMSNorm is g * x / sqrt(mean(x^2) + eps_norm) + b, per half;
  - product convention: plain bilinear, no conjugation anywhere;
  - tap W-1 of the conv multiplies the current token; no conv bias;
    history before the first token is zero unless a tail is given;
  - o_i uses the state after token i; zero initial state unless given.

Parity pins (tests/test_oracle_pins.py):
  short_conv   pinned: per-channel numpy.convolve (textbook FIR).
  silu         pinned: scipy.special.expit.
  feature_map  pinned: ||xi|| * ||y|| = 1 at eps_feat = 0; direction of y.
  feature_map_unit  pinned: ||xi|| = 1 and xi . y = ||y|| at eps_feat = 0;
               with both eps = 0 the unit-norm forward equals ||y_q|| times the
               squared one, token by token (RMSNorm removes the key-side scale).
  feature_map_rff  pinned: the values at phases 0, pi/2 and pi (order of the
               halves, sign of the sine, argument c rather than SiLU(c)),
               ||xi|| = 1, eq. 5 by Monte Carlo against the Gaussian kernel for
               Gaussian frequencies, and in the forward the identity
               xi_q . xi_k = mean_f cos(w_f^T (c_q - c_k)) with the conv outputs.
  rms_norm     pinned: mean(((z - b)/g)^2) = m/(m + eps) identity.
  zoh          pinned: quadrature of exp(lambda*tau) and scipy.linalg.expm.
  forward      pinned: O(N^2) closed form of U, O(N^3) state-free kernel form
               of o, M=1 real-EMA limit via scipy.signal.lfilter, Delta -> 0
               limit, causality, row/head independence, split-sequence resume.
  decode_step  pinned: equals the next position of a longer forward.
  forward_normalized  pinned: eta against its geometric-series closed form
               from a given start; with M = 1 and a real mode the readout is the
               ratio of two first-order IIR filters (scipy.signal.lfilter of z_v
               over lfilter of ones), whatever the queries; invariance of o
               under rescaling the query features (unit against squared map).
  forward_varlen  pinned: equal lengths give the batched forward; an empty
               sequence passes its state and tail through; a sequence split
               into two packed pieces, the second resumed from the first's
               state and tail, gives the unsplit result.
  Parity unpinned (fixed by reading only, no printed value exists): the
  complex-product convention, eps_feat and eps_norm values, the conv tap
  order, and the gain/bias shapes.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
C128 = np.complex128


def _complex(pair: np.ndarray) -> np.ndarray:
    """[..., 2] (re, im) float array -> complex128 array."""
    pair = np.asarray(pair, dtype=F64)
    return pair[..., 0] + 1j * pair[..., 1]


def zoh(log_dt, A, Bc):
    """Zero-order-hold discretisation of the per-head diagonal S4D system.

    The continuous system u'(t) = lambda u(t) + B z(t) (p1 section 2, "SSMs
    and HiPPO", with a diagonal complex A as in the S4D core of p2
    "Skalierbare Implementierung") held constant over a step of length
    Delta = exp(log_dt) gives abar = exp(Delta*lambda) and
    bbar = (exp(Delta*lambda) - 1)/lambda * B.

    log_dt [H]; A, Bc [H, M, 2] (re, im).  Returns abar, bbar complex128 [H, M].
    """
    dt = np.exp(np.asarray(log_dt, dtype=F64))[:, None]
    lam = _complex(A)
    b = _complex(Bc)
    abar = np.exp(dt * lam)
    with np.errstate(divide="ignore", invalid="ignore"):
        bbar = np.where(lam != 0, (abar - 1.0) / lam, dt) * b
    return abar, bbar


def short_conv(x, w, hist):
    """Causal depthwise short convolution SC (p2 "Skalierbare Implementierung",
    feature-map bullet: SC is a causal depthwise convolution).

    c(i)_r = sum_{j=0}^{W-1} w[h, r, j] * x(i - W + 1 + j)_r, so tap W-1 is the
    current token.  Tokens before position 0 come from hist (oldest first).

    x [B, N, H, d]; w [H, d, W]; hist [B, H, W-1, d].  Returns [B, N, H, d].
    """
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    B, N, H, d = x.shape
    W = w.shape[-1]
    hist = np.asarray(hist, dtype=F64).reshape(B, H, W - 1, d)
    xp = np.concatenate([hist.transpose(0, 2, 1, 3), x], axis=1)  # [B, N+W-1, H, d]
    c = np.zeros_like(x)
    for j in range(W):
        c += xp[:, j:j + N] * w[None, None, :, :, j]
    return c


def silu(c):
    """SiLU(c) = c * sigmoid(c) = c / (1 + exp(-c))."""
    c = np.asarray(c, dtype=F64)
    with np.errstate(over="ignore"):
        return c / (1.0 + np.exp(-c))


def feature_map(c, eps_feat):
    """xi = y / (||y||^2 + eps_feat), y = SiLU(c), norm over the last axis
    (the R channels of one head).  p2/p3 implementation bullets print the
    squared norm; eps_feat is this build's guard against an all-zero y."""
    y = silu(c)
    return y / ((y * y).sum(axis=-1, keepdims=True) + eps_feat)


def feature_map_unit(c, eps_feat):
    """Unit-norm variant xi = y / sqrt(||y||^2 + eps_feat), y = SiLU(c): the
    feature map that p1 section 1 names "SiLU/l_2", read as division by the
    plain l2 norm (the other reading of the printed squared norm)."""
    y = silu(c)
    return y / np.sqrt((y * y).sum(axis=-1, keepdims=True) + eps_feat)


def feature_map_rff(c, omega):
    """Random Fourier features xi_w(x) = [cos(w^T x), sin(w^T x)] (p1 section
    3.1, eq. 6) of the conv output x = c, with the cosine half first.  Each
    head has its own D = R/2 frequencies, the columns of omega[h] (d x D),
    drawn by the caller from the spectral density p(w) of the stationary kernel.  The
    1/sqrt(D) factor makes xi(x) . xi(x') the Monte-Carlo mean over the D
    frequencies of cos(w^T (x - x')), i.e. the estimate of K(x, x') in eq. 5.

    c [..., H, d]; omega [H, d, D].  Returns [..., H, 2D]."""
    c = np.asarray(c, dtype=F64)
    omega = np.asarray(omega, dtype=F64)
    D = omega.shape[-1]
    phase = np.einsum("...hi,hif->...hf", c, omega)
    return np.concatenate([np.cos(phase), np.sin(phase)], axis=-1) / np.sqrt(D)


FEATURE_NORMS = ("squared", "unit", "rff")


def rms_norm(x, gain, bias, eps_norm):
    """Input RMSNorm with learnable per-head gain and bias (p2 normalisation
    bullet): z = g * x / sqrt(mean(x^2) + eps_norm) + b over the last axis.

    x [B, N, H, m]; gain, bias [H, m]."""
    x = np.asarray(x, dtype=F64)
    g = np.asarray(gain, dtype=F64)[None, None]
    b = np.asarray(bias, dtype=F64)[None, None]
    return g * x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps_norm) + b


def ssm_step(U, Gamma, xi_q_i, z_k_i, z_v_i, abar, bbar):
    """One position of the shared S4D recurrence and its readout.

    The SSM input is the concatenation [z_k, z_v] (p2 recurrent-core bullet);
    both halves see the same abar, bbar.  Mode scores are the row of F_q U^T
    for this query (p1 Fig. 1 caption) and the output is the denominator-free
    readout Re(F_q U^T Gamma) (p2 last implementation bullet), read as a plain
    bilinear product without conjugation.

    U [B, H, M, R], Gamma [B, H, M, d] complex; xi_q_i, z_k_i [B, H, R];
    z_v_i [B, H, d]; abar, bbar broadcastable to [B, H, M, 1].
    Returns (U, Gamma, s [B, H, M], o_i [B, H, d]).
    """
    U = abar * U + bbar * z_k_i[:, :, None, :]
    Gamma = abar * Gamma + bbar * z_v_i[:, :, None, :]
    s = np.einsum("bhr,bhmr->bhm", xi_q_i, U)
    o_i = np.einsum("bhm,bhmc->bhc", s, Gamma).real
    return U, Gamma, s, o_i


def forward(q, k, v, params, eps_feat=1e-6, eps_norm=1e-6,
            state_in=None, tail_in=None, intermediates=False, feature_norm="squared"):
    """Forward pass of the mixer over a block of N tokens.

    q, k, v    [B, N, H, d] (any real dtype; upcast to float64)
    params     dict: conv_q, conv_k [H, d, W]; gain, bias [H, 2d] (key half
               then value half); log_dt [H]; A, Bc [H, M, 2]
    state_in   complex [B, H, M, 2d] (U then Gamma) or None (zeros)
    tail_in    [B, H, 2, W-1, d] raw q then k tokens before position 0, or None
    feature_norm  "squared" (xi = y / (||y||^2 + eps), the printed form),
               "unit" (xi = y / sqrt(||y||^2 + eps)) or "rff" (random Fourier
               features of c with params["rff_omega"] [H, d, d/2])

    Returns (o [B, N, H, d] float64, state_out complex128 [B, H, M, 2d],
    tail_out [B, H, 2, W-1, d] float64) and, with intermediates=True, a dict
    of every stage as a fourth element.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    B, N, H, d = q.shape
    W = params["conv_q"].shape[-1]
    M = params["A"].shape[1]
    gain = np.asarray(params["gain"], dtype=F64)
    bias = np.asarray(params["bias"], dtype=F64)

    if tail_in is None:
        tail_in = np.zeros((B, H, 2, W - 1, d), dtype=F64)
    tail_in = np.asarray(tail_in, dtype=F64)
    if state_in is None:
        state_in = np.zeros((B, H, M, 2 * d), dtype=C128)
    state_in = np.asarray(state_in, dtype=C128)

    # 1-2. short conv and feature map on queries and keys
    c_q = short_conv(q, params["conv_q"], tail_in[:, :, 0])
    c_k = short_conv(k, params["conv_k"], tail_in[:, :, 1])
    if feature_norm not in FEATURE_NORMS:
        raise ValueError(f"feature_norm must be one of {FEATURE_NORMS}")
    if feature_norm == "rff":
        # queries and keys share one feature space (p1 Fig. 1): the same frequencies
        xi_q = feature_map_rff(c_q, params["rff_omega"])
        xi_k = feature_map_rff(c_k, params["rff_omega"])
    else:
        fmap = feature_map if feature_norm == "squared" else feature_map_unit
        xi_q = fmap(c_q, eps_feat)
        xi_k = fmap(c_k, eps_feat)
    # 3. input RMSNorm on the key-feature half and the value half
    z_k = rms_norm(xi_k, gain[:, :d], bias[:, :d], eps_norm)
    z_v = rms_norm(v, gain[:, d:], bias[:, d:], eps_norm)
    # 4. ZOH discretisation, one (Delta, lambda, B) per head and mode
    abar, bbar = zoh(params["log_dt"], params["A"], params["Bc"])
    a4 = abar[None, :, :, None]
    b4 = bbar[None, :, :, None]

    # 5-7. recurrence over time, mode scores, readout
    U = state_in[..., :d].copy()
    Gamma = state_in[..., d:].copy()
    o = np.empty((B, N, H, d), dtype=F64)
    s_all = np.empty((B, N, H, M), dtype=C128) if intermediates else None
    for i in range(N):
        U, Gamma, s, o[:, i] = ssm_step(U, Gamma, xi_q[:, i], z_k[:, i], z_v[:, i], a4, b4)
        if intermediates:
            s_all[:, i] = s

    state_out = np.concatenate([U, Gamma], axis=-1)
    # raw tokens that precede the next block, oldest first
    qp = np.concatenate([tail_in[:, :, 0], q.transpose(0, 2, 1, 3)], axis=2)
    kp = np.concatenate([tail_in[:, :, 1], k.transpose(0, 2, 1, 3)], axis=2)
    tail_out = np.stack([qp[:, :, N:], kp[:, :, N:]], axis=2)
    if not intermediates:
        return o, state_out, tail_out
    inter = dict(c_q=c_q, c_k=c_k, xi_q=xi_q, xi_k=xi_k, z_k=z_k, z_v=z_v,
                 abar=abar, bbar=bbar, s=s_all)
    return o, state_out, tail_out, inter


def forward_normalized(q, k, v, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None,
                       eta_in=None, feature_norm="squared", parts=False):
    """Forward with the normalised readout of the derivation (p2 "Theoretische
    Herleitung" and p1 Fig. 1: the third in-loop state eta, M x 1, and the
    readout F_q U^T Gamma / (F_q U^T eta)); the scalable layer of the
    summaries drops it.  eta is read as the SSM response to a constant input
    of one, with the same abar, bbar as the other channels:
        eta_m(i) = abar_m eta_m(i-1) + bbar_m,
        o_i = Re sum_m s_m(i) Gamma_m(i) / Re sum_m s_m(i) eta_m(i),
    plain bilinear like the rest, no epsilon in the denominator.  The
    numerator is the output of forward() above.

    eta_in complex [B, H, M] or None (zeros).  Returns (o, state_out,
    tail_out, eta_out) and, with parts=True, a fifth element: a dict of num
    [B, N, H, d], den [B, N, H] and den_abs = sum_m |s_m eta_m| [B, N, H],
    the size of the terms that the denominator sums (its conditioning)."""
    num, state_out, tail_out, it = forward(q, k, v, params, eps_feat, eps_norm, state_in=state_in,
                                           tail_in=tail_in, intermediates=True, feature_norm=feature_norm)
    B, N, H, _ = num.shape
    M = it["abar"].shape[1]
    eta = np.zeros((B, H, M), dtype=C128) if eta_in is None else np.asarray(eta_in, dtype=C128).copy()
    den = np.empty((B, N, H), dtype=F64)
    den_abs = np.empty((B, N, H), dtype=F64)
    for i in range(N):
        eta = it["abar"][None] * eta + it["bbar"][None]
        den[:, i] = np.einsum("bhm,bhm->bh", it["s"][:, i], eta).real
        den_abs[:, i] = np.abs(it["s"][:, i] * eta).sum(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = num / den[..., None]
    if parts:
        return o, state_out, tail_out, eta, dict(num=num, den=den, den_abs=den_abs)
    return o, state_out, tail_out, eta


def forward_varlen(q, k, v, cu_seqlens, params, eps_feat=1e-6, eps_norm=1e-6,
                   state_in=None, tail_in=None, feature_norm="squared"):
    """Packed variable-length batch: B independent sequences laid end to end.
    Sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of the packed
    q, k, v [T, H, d]; it starts from state_in[b] and tail_in[b] (zeros when
    None) and its conv never reaches into a neighbouring sequence.  This is
    the forward above applied to each sequence on its own; a fixed-size state
    per sequence is what lets a server pack prompts of different lengths (p1
    section 1; the serving use of the fixed state).

    Returns (o [T, H, d], state_out [B, H, M, 2d], tail_out [B, H, 2, W-1, d])."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    cu = [int(x) for x in cu_seqlens]
    B = len(cu) - 1
    T, H, d = q.shape
    if cu[0] != 0 or cu[-1] != T or any(cu[b + 1] < cu[b] for b in range(B)):
        raise ValueError("cu_seqlens must rise from 0 to T")
    W = params["conv_q"].shape[-1]
    M = params["A"].shape[1]
    o = np.empty((T, H, d), dtype=F64)
    state_out = np.empty((B, H, M, 2 * d), dtype=C128)
    tail_out = np.empty((B, H, 2, W - 1, d), dtype=F64)
    for b in range(B):
        sl = slice(cu[b], cu[b + 1])
        st = None if state_in is None else np.asarray(state_in)[b:b + 1]
        tl = None if tail_in is None else np.asarray(tail_in)[b:b + 1]
        ob, state_out[b:b + 1], tail_out[b:b + 1] = forward(q[None, sl], k[None, sl], v[None, sl], params,
                                                            eps_feat, eps_norm, state_in=st, tail_in=tl,
                                                            feature_norm=feature_norm)
        o[sl] = ob[0]
    return o, state_out, tail_out


def decode_step(q_t, k_t, v_t, state, tail, params, eps_feat=1e-6, eps_norm=1e-6, feature_norm="squared"):
    """One autoregressive step: the forward pass with N = 1 from a carried
    state and conv tail (fixed-size state, O(1) work per token: p1 section 1).

    q_t, k_t, v_t [B, H, d]; state complex [B, H, M, 2d]; tail [B, H, 2, W-1, d].
    Returns (o_t [B, H, d], new state, new tail)."""
    o, st, tl = forward(np.asarray(q_t, dtype=F64)[:, None],
                        np.asarray(k_t, dtype=F64)[:, None],
                        np.asarray(v_t, dtype=F64)[:, None],
                        params, eps_feat, eps_norm, state_in=state, tail_in=tail,
                        feature_norm=feature_norm)
    return o[:, 0], st, tl
