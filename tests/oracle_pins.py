"""Pins of the fp64 oracle: each returns an error that must be ~0.

Every pin checks the oracle against something other than itself: a textbook
or library routine (numpy.convolve, scipy.special.expit, scipy.linalg.expm,
scipy.integrate.quad, scipy.signal.lfilter), an identity the definition
implies, a closed form of the recurrence, or a limit.  The functions take the
oracle module as an argument so that the mutation tests can hand in a copy
with a planted mistake and show that some pin catches it.
"""
from __future__ import annotations

import numpy as np
import scipy.integrate
import scipy.linalg
import scipy.signal
import scipy.special

import workloads as WL


def rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    den = max(float(np.linalg.norm(b)), 1e-300)
    return float(np.linalg.norm(a - b)) / den


def pin_case(seed=11, B=2, N=40, H=2, d=6, M=5, W=4, with_state=False):
    """A small case whose parameters are spread out so that every term of the
    method moves the output: random gains, larger biases, larger Delta, random
    complex lambda (Re < 0) and complex B, nonzero conv history."""
    s = WL.spec("tiny", tag=97, B=B, N=N, H=H, d=d, M=M, W=W)
    p = WL.make_params(s, seed)
    q, k, v = WL.make_rows(s, seed=seed)
    r = np.random.default_rng(1000 + seed)
    p["gain"] = r.uniform(0.5, 1.5, (H, 2 * d))
    p["bias"] = r.normal(0.0, 0.3, (H, 2 * d))
    p["log_dt"] = np.log(r.uniform(0.05, 0.4, H))
    A = np.empty((H, M, 2))
    A[..., 0] = -r.uniform(0.1, 1.0, (H, M))
    A[..., 1] = r.normal(0.0, 3.0, (H, M))
    Bc = np.empty((H, M, 2))
    Bc[..., 0] = r.normal(1.0, 0.3, (H, M))
    Bc[..., 1] = r.normal(0.0, 0.5, (H, M))
    p["A"], p["Bc"] = A, Bc
    tail = r.normal(size=(B, H, 2, W - 1, d))
    state = None
    if with_state:
        state = 0.3 * (r.normal(size=(B, H, M, 2 * d)) + 1j * r.normal(size=(B, H, M, 2 * d)))
    return dict(p=p, q=q, k=k, v=v, tail=tail, state=state)


# ------------------------------------------------------------------ stages
def pin_conv(O) -> float:
    """short_conv against per-channel numpy.convolve of the causal filter whose
    lag-0 tap is w[..., W-1]."""
    r = np.random.default_rng(5)
    B, N, H, d, W = 2, 23, 3, 4, 4
    x = r.normal(size=(B, N, H, d))
    w = r.normal(size=(H, d, W))
    hist = r.normal(size=(B, H, W - 1, d))
    got = O.short_conv(x, w, hist)
    ref = np.empty_like(got)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                full = np.concatenate([hist[b, h, :, c], x[b, :, h, c]])
                ref[b, :, h, c] = np.convolve(full, w[h, c, ::-1], mode="valid")
    return rel(got, ref)


def pin_silu(O) -> float:
    c = np.linspace(-30, 30, 1201)
    return rel(O.silu(c), c * scipy.special.expit(c))


def pin_feature_map(O) -> float:
    """With eps_feat = 0: xi . y = 1 and ||xi|| ||y|| = 1, which together force
    xi = y / ||y||^2 (Cauchy-Schwarz equality)."""
    r = np.random.default_rng(6)
    c = r.normal(size=(3, 7, 2, 16)) * 2.0
    y = c * scipy.special.expit(c)
    xi = O.feature_map(c, 0.0)
    dot = (xi * y).sum(-1)
    nn = np.linalg.norm(xi, axis=-1) * np.linalg.norm(y, axis=-1)
    return max(float(np.abs(dot - 1).max()), float(np.abs(nn - 1).max()))


def pin_feature_map_unit(O) -> float:
    """With eps_feat = 0: ||xi|| = 1 and xi . y = ||y||, which together force
    xi = y / ||y|| (Cauchy-Schwarz equality)."""
    r = np.random.default_rng(16)
    c = r.normal(size=(3, 7, 2, 16)) * 2.0
    y = c * scipy.special.expit(c)
    xi = O.feature_map_unit(c, 0.0)
    ny = np.linalg.norm(y, axis=-1)
    e1 = np.abs(np.linalg.norm(xi, axis=-1) - 1).max()
    e2 = np.abs((xi * y).sum(-1) - ny).max() / ny.max()
    return max(float(e1), float(e2))


def pin_rff_special(O) -> float:
    """Random Fourier features at phases where cos and sin are exact: x = 0
    gives [1, ..., 1, 0, ..., 0]/sqrt(D) (cosine half first); x = e_0 with every
    frequency's first entry pi/2 gives [0, ..., 0, 1, ..., 1]/sqrt(D) (sin
    taken with a plus sign, of x itself and not of SiLU(x)); entries pi give
    [-1, ..., -1, 0, ..., 0]/sqrt(D)."""
    r = np.random.default_rng(21)
    H, d, D = 2, 8, 4
    omega = r.normal(size=(H, d, D))
    x = np.zeros((3, H, d))
    x[1:, :, 0] = 1.0
    omega[:, 0, :] = np.pi / 2
    want = np.zeros((3, H, 2 * D))
    want[0, :, :D] = 1.0
    want[1, :, D:] = 1.0
    xi = O.feature_map_rff(x[:2], omega)
    omega[:, 0, :] = np.pi
    want[2, :, :D] = -1.0
    xi = np.concatenate([xi, O.feature_map_rff(x[2:], omega)])
    return float(np.abs(xi - want / np.sqrt(D)).max())


def pin_rff_norm(O) -> float:
    """||xi(x)|| = 1 for every x (cos^2 + sin^2 = 1, D terms of 1/D)."""
    r = np.random.default_rng(22)
    xi = O.feature_map_rff(r.normal(size=(5, 6, 3, 16)) * 3, r.normal(size=(3, 16, 8)))
    return float(np.abs(np.linalg.norm(xi, axis=-1) - 1).max())


def pin_rff_bochner(O) -> float:
    """p1 eq. 5: with frequencies w ~ N(0, I / sigma^2), the mean of
    xi(x) . xi(x') over many frequencies estimates the Gaussian kernel
    exp(-||x - x'||^2 / (2 sigma^2)), the Fourier transform of that density.
    D = 40000 frequencies: the Monte-Carlo standard error is below 0.004, so
    the returned error is divided by 0.02 (the pin's tolerance is 1)."""
    r = np.random.default_rng(23)
    d, D, sigma = 5, 40000, 1.3
    omega = r.normal(size=(1, d, D)) / sigma
    x = r.normal(size=(6, 1, d)) * 0.8
    xi = O.feature_map_rff(x, omega)[:, 0]
    est = xi @ xi.T
    dist2 = ((x[:, None, 0] - x[None, :, 0]) ** 2).sum(-1)
    return float(np.abs(est - np.exp(-dist2 / (2 * sigma * sigma))).max() / 0.02)


def pin_rff_wiring(O) -> float:
    """In the forward with the RFF map, queries and keys use the same
    frequencies on the conv outputs: xi_q(i) . xi_k(j) equals
    mean_f cos(w_f^T (c_q(i) - c_k(j))) for every pair of positions."""
    c = pin_case()
    p = dict(c["p"])
    H, d = c["q"].shape[2], c["q"].shape[3]
    p["rff_omega"] = np.random.default_rng(24).normal(size=(H, d, d // 2))
    _, _, _, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True, feature_norm="rff")
    err = 0.0
    for h in range(H):
        dots = np.einsum("bih,bjh->bij", it["xi_q"][:, :, h], it["xi_k"][:, :, h])
        diff = it["c_q"][:, :, None, h] - it["c_k"][:, None, :, h]          # [B, N, N, d]
        want = np.cos(np.einsum("bijc,cf->bijf", diff, p["rff_omega"][h])).mean(-1)
        err = max(err, float(np.abs(dots - want).max()))
    return err


def pin_unit_scaling(O) -> float:
    """With eps_feat = eps_norm = 0 the key features enter only through RMSNorm,
    which is blind to a per-token scale, and the query features scale s (hence
    o) by ||y_q||: o_unit(i) = ||SiLU(SC(q))(i)|| o_squared(i), per token and
    head.  The norm comes from scipy.special.expit and the oracle's conv, which
    the conv pin ties to numpy.convolve."""
    c = pin_case(with_state=True)
    q, k, v, p = c["q"], c["k"], c["v"], c["p"]
    o_sq = O.forward(q, k, v, p, 0.0, 0.0, c["state"], c["tail"])[0]
    o_un = O.forward(q, k, v, p, 0.0, 0.0, c["state"], c["tail"], feature_norm="unit")[0]
    cq = O.short_conv(q, p["conv_q"], np.asarray(c["tail"])[:, :, 0])
    ny = np.linalg.norm(cq * scipy.special.expit(cq), axis=-1, keepdims=True)
    return rel(o_un, ny * o_sq)


def pin_rms_norm(O) -> float:
    """((z - b)/g) is parallel to x with mean square m/(m + eps)."""
    r = np.random.default_rng(7)
    x = r.normal(size=(2, 9, 3, 12)) * r.uniform(0.01, 3.0, size=(2, 9, 3, 1))
    g = r.uniform(0.5, 1.5, size=(3, 12))
    b = r.normal(size=(3, 12))
    eps = 1e-3
    z = O.rms_norm(x, g, b, eps)
    u = (z - b[None, None]) / g[None, None]
    m = (x * x).mean(-1)
    e1 = np.abs((u * u).mean(-1) - m / (m + eps)).max()
    cos = (u * x).sum(-1) / (np.linalg.norm(u, axis=-1) * np.linalg.norm(x, axis=-1))
    return max(float(e1), float(np.abs(cos - 1).max()))


def pin_zoh(O) -> float:
    """abar against expm of the 2x2 real form of lambda; bbar against the
    Van Loan block exponential expm([[A dt, B dt], [0, 0]]) and against
    quadrature of int_0^dt exp(lambda tau) d tau * B."""
    r = np.random.default_rng(8)
    H, M = 3, 4
    log_dt = np.log(r.uniform(1e-3, 0.5, H))
    A = np.stack([-r.uniform(0.05, 2.0, (H, M)), r.normal(0, 10, (H, M))], -1)
    Bc = np.stack([r.normal(1, 0.3, (H, M)), r.normal(0, 0.5, (H, M))], -1)
    abar, bbar = O.zoh(log_dt, A, Bc)
    err = 0.0
    for h in range(H):
        dt = np.exp(log_dt[h])
        for m in range(M):
            a, w = A[h, m]
            A2 = np.array([[a, -w], [w, a]])
            big = np.zeros((3, 3))
            big[:2, :2] = A2 * dt
            big[:2, 2] = Bc[h, m] * dt
            E = scipy.linalg.expm(big)
            ab = E[0, 0] + 1j * E[1, 0]
            bb = E[0, 2] + 1j * E[1, 2]
            lam = a + 1j * w
            re = scipy.integrate.quad(lambda t: np.exp(lam * t).real, 0, dt, epsabs=0, epsrel=1e-13)[0]
            im = scipy.integrate.quad(lambda t: np.exp(lam * t).imag, 0, dt, epsabs=0, epsrel=1e-13)[0]
            bq = (re + 1j * im) * (Bc[h, m, 0] + 1j * Bc[h, m, 1])
            err = max(err, abs(abar[h, m] - ab) / abs(ab), abs(bbar[h, m] - bb) / abs(bb),
                      abs(bbar[h, m] - bq) / abs(bq))
    return float(err)


def pin_wiring(O) -> float:
    """Stage outputs of forward satisfy the stage identities with the
    documented operands: q-conv weights on q, key half of gain/bias on xi_k,
    value half on v, the given tail as conv history."""
    c = pin_case()
    p = c["p"]
    o, st, tl, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-4, None, c["tail"], True)
    d = c["q"].shape[-1]
    errs = []
    for x, w, hist, name in ((c["q"], p["conv_q"], c["tail"][:, :, 0], "c_q"),
                            (c["k"], p["conv_k"], c["tail"][:, :, 1], "c_k")):
        B, N, H, _ = x.shape
        ref = np.empty((B, N, H, d))
        for b in range(B):
            for h in range(H):
                for ch in range(d):
                    full = np.concatenate([hist[b, h, :, ch], x[b, :, h, ch]])
                    ref[b, :, h, ch] = np.convolve(full, w[h, ch, ::-1], mode="valid")
        errs.append(rel(it[name], ref))
    for cn, xn in (("c_q", "xi_q"), ("c_k", "xi_k")):
        y = it[cn] * scipy.special.expit(it[cn])
        ysq = (y * y).sum(-1)
        errs.append(float(np.abs((it[xn] * y).sum(-1) * (ysq + 1e-6) / ysq - 1).max()))
    for z, x, sl in (("z_k", it["xi_k"], slice(0, d)), ("z_v", np.asarray(c["v"], float), slice(d, 2 * d))):
        g = np.asarray(p["gain"])[:, sl][None, None]
        b = np.asarray(p["bias"])[:, sl][None, None]
        u = (it[z] - b) / g
        m = (x * x).mean(-1)
        errs.append(float(np.abs((u * u).mean(-1) - m / (m + 1e-4)).max() / np.abs(m / (m + 1e-4)).max()))
        cos = (u * x).sum(-1) / (np.linalg.norm(u, axis=-1) * np.linalg.norm(x, axis=-1))
        errs.append(float(np.abs(cos - 1).max()))
    return max(errs)


# ------------------------------------------------------------------ recurrence
def pin_closed_form(O, with_state=True) -> float:
    """O(N^2) closed form of the recurrence:
    U_m(i) = abar^(i+1) U_m(-1) + sum_{j<=i} abar^(i-j) bbar z_k(j), likewise
    Gamma; then s_m(i) = xi_q(i) . U_m(i) and o_i = Re sum_m s_m(i) Gamma_m(i)."""
    c = pin_case(with_state=with_state)
    p = c["p"]
    o, st, tl, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, c["state"], c["tail"], True)
    B, N, H, d = o.shape
    abar, bbar = O.zoh(p["log_dt"], p["A"], p["Bc"])
    M = abar.shape[1]
    st0 = c["state"] if c["state"] is not None else np.zeros((B, H, M, 2 * d), complex)
    s_ref = np.empty((B, N, H, M), complex)
    o_ref = np.empty((B, N, H, d))
    for i in range(N):
        t = np.arange(i + 1)
        pw = abar[:, :, None] ** (i - t)[None, None, :]                 # [H, M, i+1]
        U = np.einsum("hmj,bjhr->bhmr", pw * bbar[:, :, None], it["z_k"][:, :i + 1])
        G = np.einsum("hmj,bjhr->bhmr", pw * bbar[:, :, None], it["z_v"][:, :i + 1])
        U = U + (abar ** (i + 1))[None, :, :, None] * st0[..., :d]
        G = G + (abar ** (i + 1))[None, :, :, None] * st0[..., d:]
        s_ref[:, i] = np.einsum("bhr,bhmr->bhm", it["xi_q"][:, i], U)
        o_ref[:, i] = np.einsum("bhm,bhmc->bhc", s_ref[:, i], G).real
        if i == N - 1:
            st_ref = np.concatenate([U, G], -1)
    return max(rel(it["s"], s_ref), rel(o, o_ref), rel(st, st_ref))


def pin_kernel_form(O) -> float:
    """State-free O(N^3) form: o_i = sum_{j,l<=i} (xi_q(i).z_k(j)) K(2i-j-l) z_v(l)
    with K(t) = Re sum_m bbar_m^2 abar_m^t.  It follows from the plain
    bilinear readout because abar^(i-j) abar^(i-l) = abar^(2i-j-l); a
    conjugated product or swapped operands give a different kernel."""
    c = pin_case(N=24)
    p = c["p"]
    o, st, tl, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True)
    B, N, H, d = o.shape
    abar, bbar = O.zoh(p["log_dt"], p["A"], p["Bc"])
    tmax = 2 * N
    K = np.einsum("hm,hmt->ht", bbar ** 2, abar[:, :, None] ** np.arange(tmax)[None, None]).real  # [H, t]
    o_ref = np.zeros_like(o)
    for i in range(N):
        j = np.arange(i + 1)
        gram = np.einsum("bhr,bjhr->bhj", it["xi_q"][:, i], it["z_k"][:, :i + 1])   # [B,H,j]
        T = 2 * i - j[:, None] - j[None, :]                                           # [j, l]
        Kij = K[:, T]                                                                 # [H, j, l]
        o_ref[:, i] = np.einsum("bhj,hjl,blhc->bhc", gram, Kij, it["z_v"][:, :i + 1])
    return rel(o, o_ref)


def pin_m1_lfilter(O) -> float:
    """M = 1 with a real lambda: U and Gamma are real first-order IIR filters
    of z_k and z_v, u = lfilter([bbar], [1, -abar], z), so o = (xi_q . u) gamma."""
    c = pin_case(M=1, N=60)
    p = c["p"]
    p["A"] = np.array(p["A"])
    p["A"][..., 1] = 0.0
    p["Bc"] = np.array(p["Bc"])
    p["Bc"][..., 1] = 0.0
    o, st, tl, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True)
    dt = np.exp(np.asarray(p["log_dt"], float))
    lam = np.asarray(p["A"], float)[:, 0, 0]
    ab = np.exp(dt * lam)
    bb = (ab - 1) / lam * np.asarray(p["Bc"], float)[:, 0, 0]
    o_ref = np.empty_like(o)
    for h in range(o.shape[2]):
        u = scipy.signal.lfilter([bb[h]], [1.0, -ab[h]], it["z_k"][:, :, h], axis=1)
        g = scipy.signal.lfilter([bb[h]], [1.0, -ab[h]], it["z_v"][:, :, h], axis=1)
        o_ref[:, :, h] = (it["xi_q"][:, :, h] * u).sum(-1, keepdims=True) * g
    return rel(o, o_ref)


def pin_eta_closed_form(O) -> float:
    """The normaliser state from a start eta0 after n tokens is the geometric
    series abar^n eta0 + bbar (1 - abar^n) / (1 - abar)."""
    c = pin_case(with_state=True)
    p = c["p"]
    B, N, H, _ = c["q"].shape
    M = np.asarray(p["A"]).shape[1]
    eta0 = np.random.default_rng(31).normal(size=(B, H, M)) + 1j * np.random.default_rng(32).normal(size=(B, H, M))
    _, _, _, eta = O.forward_normalized(c["q"], c["k"], c["v"], p, state_in=c["state"], tail_in=c["tail"],
                                        eta_in=eta0)
    dt = np.exp(np.asarray(p["log_dt"], float))[:, None]
    lam = np.asarray(p["A"], float)[..., 0] + 1j * np.asarray(p["A"], float)[..., 1]
    bc = np.asarray(p["Bc"], float)[..., 0] + 1j * np.asarray(p["Bc"], float)[..., 1]
    abar = np.exp(dt * lam)
    bbar = (abar - 1) / lam * bc
    want = abar[None] ** N * eta0 + bbar[None] * (1 - abar[None] ** N) / (1 - abar[None])
    return rel(eta, want)


def pin_eta_m1_ratio(O) -> float:
    """M = 1 with a real mode: s is a scalar per token that multiplies both
    Gamma and eta, so o = lfilter(z_v) / lfilter(ones), the ratio of two
    first-order IIR filters, whatever the queries."""
    c = pin_case(M=1, N=60)
    p = c["p"]
    p["A"] = np.array(p["A"])
    p["A"][..., 1] = 0.0
    p["Bc"] = np.array(p["Bc"])
    p["Bc"][..., 1] = 0.0
    o, _, _, _ = O.forward_normalized(c["q"], c["k"], c["v"], p, tail_in=c["tail"])
    _, _, _, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True)
    dt = np.exp(np.asarray(p["log_dt"], float))
    lam = np.asarray(p["A"], float)[:, 0, 0]
    ab = np.exp(dt * lam)
    bb = (ab - 1) / lam * np.asarray(p["Bc"], float)[:, 0, 0]
    o_ref = np.empty_like(o)
    for h in range(o.shape[2]):
        g = scipy.signal.lfilter([bb[h]], [1.0, -ab[h]], it["z_v"][:, :, h], axis=1)
        e = scipy.signal.lfilter([bb[h]], [1.0, -ab[h]], np.ones(o.shape[1]))
        o_ref[:, :, h] = g / e[None, :, None]
    return rel(o, o_ref)


def pin_eta_kernel_form(O) -> float:
    """State-free form of the normalised readout's denominator:
    den(i) = sum_{j,l<=i} (xi_q(i).z_k(j)) K(2i-j-l) with the same kernel
    K(t) = Re sum_m bbar_m^2 abar_m^t as the numerator's (z_v(l) replaced by
    the constant input 1).  A conjugated product gives another kernel."""
    c = pin_case(N=24)
    p = c["p"]
    o, _, _, _, pt = O.forward_normalized(c["q"], c["k"], c["v"], p, tail_in=c["tail"], parts=True)
    num, den = pt["num"], pt["den"]
    _, _, _, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True)
    B, N, H, d = o.shape
    abar, bbar = O.zoh(p["log_dt"], p["A"], p["Bc"])
    K = np.einsum("hm,hmt->ht", bbar ** 2, abar[:, :, None] ** np.arange(2 * N)[None, None]).real
    den_ref = np.zeros((B, N, H))
    for i in range(N):
        j = np.arange(i + 1)
        gram = np.einsum("bhr,bjhr->bhj", it["xi_q"][:, i], it["z_k"][:, :i + 1])
        den_ref[:, i] = np.einsum("bhj,hjl->bh", gram, K[:, 2 * i - j[:, None] - j[None, :]])
    return max(rel(den, den_ref), rel(o * den[..., None], num))


def pin_eta_query_scale(O) -> float:
    """The normalised readout does not depend on the scale of the query
    features: with eps = 0 the unit-norm and the squared map (which differ by
    the factor ||y_q|| per token) give the same o."""
    c = pin_case(with_state=True)
    args = (c["q"], c["k"], c["v"], c["p"], 0.0, 0.0, c["state"], c["tail"])
    o_sq = O.forward_normalized(*args, feature_norm="squared")[0]
    o_un = O.forward_normalized(*args, feature_norm="unit")[0]
    return rel(o_un, o_sq)


def pin_dt_zero(O) -> float:
    """Delta -> 0: abar -> 1, bbar -> Delta B, so
    o_i / Delta^2 -> (sum_m B_m^2) (xi_q(i) . sum_{j<=i} z_k(j)) sum_{l<=i} z_v(l).
    The first-order correction is about Delta * N * |Re lambda| ~ 1e-6 here."""
    c = pin_case(N=64)
    p = c["p"]
    dt = 1e-8
    p["log_dt"] = np.full(p["log_dt"].shape, np.log(dt))
    p["Bc"] = np.array(p["Bc"])
    p["Bc"][..., 1] = 0.0
    o, st, tl, it = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, None, c["tail"], True)
    sumB2 = (np.asarray(p["Bc"], float)[..., 0] ** 2).sum(-1)     # [H]
    Zk = np.cumsum(it["z_k"], axis=1)
    Zv = np.cumsum(it["z_v"], axis=1)
    ref = sumB2[None, None, :, None] * (it["xi_q"] * Zk).sum(-1, keepdims=True) * Zv
    return rel(o / dt ** 2, ref)


# ------------------------------------------------------------------ invariants
def pin_causality(O) -> float:
    c = pin_case()
    o1 = O.forward(c["q"], c["k"], c["v"], c["p"], tail_in=c["tail"])[0]
    q2, k2, v2 = (np.array(x, float) for x in (c["q"], c["k"], c["v"]))
    cut = 17
    for x in (q2, k2, v2):
        x[:, cut:] += 5.0
    o2 = O.forward(q2, k2, v2, c["p"], tail_in=c["tail"])[0]
    return float(np.abs(o1[:, :cut] - o2[:, :cut]).max())


def pin_split_resume(O) -> float:
    """forward(x) equals forward(x[:n1]) followed by forward(x[n1:]) resumed
    from the first call's state and tail; also at a split shorter than W-1."""
    c = pin_case(with_state=True)
    q, k, v, p = c["q"], c["k"], c["v"], c["p"]
    o, st, tl = O.forward(q, k, v, p, state_in=c["state"], tail_in=c["tail"])
    err = 0.0
    for n1 in (1, 2, 13):
        oa, sa, ta = O.forward(q[:, :n1], k[:, :n1], v[:, :n1], p, state_in=c["state"], tail_in=c["tail"])
        ob, sb, tb = O.forward(q[:, n1:], k[:, n1:], v[:, n1:], p, state_in=sa, tail_in=ta)
        err = max(err, rel(np.concatenate([oa, ob], 1), o), rel(sb, st), rel(tb, tl))
    return err


def pin_decode(O) -> float:
    """decode_step from the state and tail after n tokens equals position n of
    the forward over n+1 tokens."""
    c = pin_case(with_state=True)
    q, k, v, p = c["q"], c["k"], c["v"], c["p"]
    n = q.shape[1] - 1
    o, st, tl = O.forward(q, k, v, p, state_in=c["state"], tail_in=c["tail"])
    _, sa, ta = O.forward(q[:, :n], k[:, :n], v[:, :n], p, state_in=c["state"], tail_in=c["tail"])
    ot, sn, tn = O.decode_step(q[:, n], k[:, n], v[:, n], sa, ta, p)
    return max(rel(ot, o[:, n]), rel(sn, st), rel(tn, tl))


def pin_independence(O) -> float:
    """Batch rows and heads do not interact."""
    c = pin_case(B=3, H=3)
    q, k, v, p = c["q"], c["k"], c["v"], c["p"]
    o = O.forward(q, k, v, p, tail_in=c["tail"])[0]
    o_row = O.forward(q[1:2], k[1:2], v[1:2], p, tail_in=c["tail"][1:2])[0]
    ph = {key: np.asarray(val)[2:3] for key, val in p.items()}
    o_head = O.forward(q[:, :, 2:3], k[:, :, 2:3], v[:, :, 2:3], ph, tail_in=c["tail"][:, 2:3])[0]
    return max(rel(o_row, o[1:2]), rel(o_head, o[:, :, 2:3]))


def pin_varlen(O) -> float:
    """Packed variable-length batches: (a) equal lengths equal the batched
    forward of the same rows; (b) a zero-length sequence returns its state and
    tail unchanged; (c) one row cut into two packed pieces, the second
    resumed from the first's end state and tail, equals the row in one piece;
    (d) no output leaks between neighbouring sequences (changing one
    sequence's tokens leaves the others' outputs bit-identical)."""
    c = pin_case(with_state=True)
    p = c["p"]
    B, N, H, d = c["q"].shape
    st, tl = c["state"], c["tail"]
    o, so, to = O.forward(c["q"], c["k"], c["v"], p, state_in=st, tail_in=tl)
    pack = lambda x: x.reshape(B * N, H, d)
    cu = [b * N for b in range(B + 1)]
    ov, sv, tv = O.forward_varlen(pack(c["q"]), pack(c["k"]), pack(c["v"]), cu, p, state_in=st, tail_in=tl)
    errs = [rel(ov.reshape(B, N, H, d), o), rel(sv, so), rel(tv, to)]
    # (b) empty first sequence, then row 0 whole
    cu2 = [0, 0, N]
    st2 = np.concatenate([st[1:2], st[0:1]])
    tl2 = np.concatenate([tl[1:2], tl[0:1]])
    o2, s2, t2 = O.forward_varlen(c["q"][0], c["k"][0], c["v"][0], cu2, p, state_in=st2, tail_in=tl2)
    errs += [rel(s2[0], st[1]), rel(t2[0], tl[1]), rel(o2, o[0]), rel(s2[1], so[0])]
    # (c) row 0 cut at n1 into two sequences of one packed batch: the second piece
    # resumes from the first's end state and tail
    n1 = 13
    a_o, a_s, a_t = O.forward_varlen(c["q"][0, :n1], c["k"][0, :n1], c["v"][0, :n1], [0, n1], p,
                                     state_in=st[:1], tail_in=tl[:1])
    cu3 = [0, n1, N]
    st3 = np.concatenate([st[:1], a_s])
    tl3 = np.concatenate([tl[:1], a_t])
    o3, s3, t3 = O.forward_varlen(c["q"][0], c["k"][0], c["v"][0], cu3, p, state_in=st3, tail_in=tl3)
    errs += [rel(o3, o[0]), rel(s3[1], so[0]), rel(t3[1], to[0])]
    # (d) isolation
    q4 = pack(c["q"]).copy()
    q4[N:] += 1.0
    o4, _, _ = O.forward_varlen(q4, pack(c["k"]), pack(c["v"]), cu, p, state_in=st, tail_in=tl)
    errs.append(float(np.abs(o4[:N] - ov[:N]).max()))
    return max(errs)


def pin_backward_forward_torch(O) -> float:
    """The differentiable torch forward of the backward oracle equals the
    NumPy oracle's forward (output and end state), for every feature map."""
    from oracle import idattn_backward as BW
    c = pin_case(with_state=True)
    p = dict(c["p"])
    H, d = c["q"].shape[2], c["q"].shape[3]
    p["rff_omega"] = np.random.default_rng(41).normal(size=(H, d, d // 2))
    err = 0.0
    for fm in ("squared", "unit", "rff"):
        o, st, _ = O.forward(c["q"], c["k"], c["v"], p, 1e-6, 1e-6, c["state"], c["tail"], feature_norm=fm)
        pt = {k: torch_t(v) for k, v in p.items()}
        ot, stt = BW.forward_torch(torch_t(c["q"]), torch_t(c["k"]), torch_t(c["v"]), pt, 1e-6, 1e-6,
                                   torch_c(c["state"]), torch_t(c["tail"]), fm)
        err = max(err, rel(ot.numpy(), o), rel(stt.numpy(), st))
    return err


def torch_t(x):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def torch_c(z):
    import torch
    return torch.as_tensor(np.asarray(z, dtype=np.complex128))


def pin_backward_finite_differences(O) -> float:
    """Directional derivatives of L = sum(g_o * o) + Re sum(conj(g_s) * state_out)
    from the backward oracle against central differences of the NumPy
    forward, along a random direction in each input: q, k, v, every parameter
    and the carried state.  Returns the largest relative mismatch."""
    from oracle import idattn_backward as BW
    c = pin_case(with_state=True, N=12)
    p = c["p"]
    r = np.random.default_rng(42)
    g_o = r.normal(size=c["q"].shape)
    g_s = r.normal(size=c["state"].shape) + 1j * r.normal(size=c["state"].shape)

    def loss(q, k, v, pp, st):
        o, so, _ = O.forward(q, k, v, pp, 1e-6, 1e-6, st, c["tail"])
        return float((g_o * o).sum() + (np.conj(g_s) * so).real.sum())

    grads = BW.backward(c["q"], c["k"], c["v"], p, g_o, 1e-6, 1e-6, c["state"], c["tail"], g_s)
    h = 1e-5
    worst = 0.0
    names = ["q", "k", "v"] + list(BW.PARAM_KEYS) + ["state"]
    for name in names:
        base = c["state"] if name == "state" else (c[name] if name in ("q", "k", "v") else p[name])
        base = np.asarray(base)
        delta = r.normal(size=base.shape)
        if name == "state":
            delta = delta + 1j * r.normal(size=base.shape)

        def at(x):
            args = dict(q=c["q"], k=c["k"], v=c["v"], st=c["state"])
            pp = dict(p)
            if name in ("q", "k", "v"):
                args[name] = x
            elif name == "state":
                args["st"] = x
            else:
                pp[name] = x
            return loss(args["q"], args["k"], args["v"], pp, args["st"])

        fd = (at(base + h * delta) - at(base - h * delta)) / (2 * h)
        an = float((np.conj(grads[name]) * delta).real.sum()) if name == "state" else float((grads[name] * delta).sum())
        worst = max(worst, abs(an - fd) / max(abs(fd), 1e-12))
    return worst


PINS = {
    "conv": (pin_conv, 1e-13),
    "silu": (pin_silu, 1e-14),
    "feature_map": (pin_feature_map, 1e-12),
    "feature_map_unit": (pin_feature_map_unit, 1e-12),
    "unit_scaling": (pin_unit_scaling, 1e-11),
    "rff_special": (pin_rff_special, 1e-15),
    "rff_norm": (pin_rff_norm, 1e-14),
    "rff_bochner": (pin_rff_bochner, 1.0),
    "rff_wiring": (pin_rff_wiring, 1e-13),
    "rms_norm": (pin_rms_norm, 1e-12),
    "zoh": (pin_zoh, 1e-10),
    "wiring": (pin_wiring, 1e-10),
    "closed_form": (pin_closed_form, 1e-12),
    "kernel_form": (pin_kernel_form, 1e-11),
    "m1_lfilter": (pin_m1_lfilter, 1e-12),
    "dt_zero": (pin_dt_zero, 1e-5),
    "causality": (pin_causality, 0.0),
    "split_resume": (pin_split_resume, 1e-12),
    "decode": (pin_decode, 1e-12),
    "varlen": (pin_varlen, 1e-12),
    "backward_forward_torch": (pin_backward_forward_torch, 1e-12),
    "backward_finite_differences": (pin_backward_finite_differences, 1e-6),
    "eta_closed_form": (pin_eta_closed_form, 1e-12),
    "eta_m1_ratio": (pin_eta_m1_ratio, 1e-11),
    "eta_query_scale": (pin_eta_query_scale, 1e-10),
    "eta_kernel_form": (pin_eta_kernel_form, 1e-11),
    "independence": (pin_independence, 1e-13),
}
