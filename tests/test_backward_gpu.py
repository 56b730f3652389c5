"""GPU parity of idattn_backward against the fp64 autograd oracle
(oracle/idattn_backward.py, itself pinned by finite differences of the NumPy
forward): every gradient, q, k, v, each parameter and the carried state.

Gates (relative L2): input gradients in the I/O dtype at 1e-5 (fp32) and
2e-3 (bf16: the rounding of the stored gradient alone costs about 1.7e-3),
whole tensor and per (b, h); parameter and state gradients are fp32 outputs
of fp32 arithmetic on the same stored values, at 1e-5 in both modes."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as WL
from tests.gpu_util import GATE_BF16, GATE_F32, check, down, state_dev, state_np, up

pytestmark = pytest.mark.gpu

PARAM_KEYS = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc")


@pytest.fixture(scope="module")
def fs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fixed_state_ssm_amd as fs
    fs.load_library()
    return fs


def _sync():
    import torch
    torch.cuda.synchronize()


def _grad_inputs(s, seed):
    """grad_o [B, N, H, d] (stored values) and grad_state complex [B, H, M, 2d]."""
    r = np.random.default_rng(seed)
    go = r.standard_normal((s["B"], s["N"], s["H"], s["d"])).astype(np.float32)
    if s["io"] == "bf16":
        go = WL.bf16_round(go)
    gS = (0.1 * (r.standard_normal((s["B"], s["H"], s["M"], 2 * s["d"]))
                 + 1j * r.standard_normal((s["B"], s["H"], s["M"], 2 * s["d"])))).astype(np.complex64)
    return go, gS


def _log_dt_term_scale(params, want):
    """Per head, sum_m of the magnitudes of the terms whose sum is the log_dt
    gradient, Delta Re(conj(lambda abar) g_abar + conj(B abar) g_bbar).
    g_abar and g_bbar are recovered from the oracle's own lambda and B
    gradients through the ZOH chain rule:
      g_B = conj((abar - 1)/lambda) g_bbar,
      g_lambda = conj(Delta abar) g_abar + conj(B Delta^2 phi(Delta lambda)) g_bbar,
      phi(z) = (exp(z)(z - 1) + 1)/z^2 (its series for small z)."""
    dt = np.exp(np.asarray(params["log_dt"], np.float64))[:, None]
    A = np.asarray(params["A"], np.float64)
    Bc = np.asarray(params["Bc"], np.float64)
    lam, bc = A[..., 0] + 1j * A[..., 1], Bc[..., 0] + 1j * Bc[..., 1]
    z = dt * lam
    abar = np.exp(z)
    q = np.where(lam != 0, np.expm1(z) / np.where(lam != 0, lam, 1), dt)
    small = np.abs(z) < 0.5
    series = sum(z ** (n - 2) * (n - 1) / np.prod(np.arange(1, n + 1, dtype=np.float64)) for n in range(2, 30))
    zz = np.where(small, 1.0, z)
    phi = np.where(small, series, (np.exp(zz) * (zz - 1) + 1) / zz ** 2)
    gl = want["A"][..., 0] + 1j * want["A"][..., 1]
    gB = want["Bc"][..., 0] + 1j * want["Bc"][..., 1]
    gbb = gB / np.conj(q)
    gab = (gl - np.conj(bc * dt ** 2 * phi) * gbb) / np.conj(dt * abar)
    return (dt * (np.abs(lam * abar * gab) + np.abs(bc * abar * gbb))).sum(-1)


def _compare(tag, got, want, io, params, pgate=GATE_F32):
    g_in = GATE_BF16 if io == "bf16" else GATE_F32
    for key in ("q", "k", "v"):
        check(f"{tag} grad {key}", down(got[key]), want[key], g_in, io)
    for key in PARAM_KEYS:
        g = got[key].cpu().numpy().astype(np.float64)
        if key == "log_dt":
            # a per-head sum over modes of terms of both signs: its rounding
            # error scales with the terms, not with the (smaller) sum
            scale = _log_dt_term_scale(params, want)
            ratio = float((np.abs(g - want[key]) / (pgate * scale)).max())
            print(f"{tag} grad log_dt: relL2 {np.linalg.norm(g - want[key]) / np.linalg.norm(want[key]):.3e}, "
                  f"error / (gate x sum of term magnitudes) {ratio:.3f}", flush=True)
            assert ratio <= 1.0, (tag, ratio)
            continue
        check(f"{tag} grad {key}", g, want[key], pgate, pairs=False)
    if "state" in want:
        check(f"{tag} grad state_in", state_np(got["state"]), want["state"], pgate, io)


# name: (base config, overrides, seed tag, feature map)
BWD = {
    "tiny_f32": ("tiny", {}, 101, "squared"),
    "d32_m64_w2_f32": ("tiny", dict(d=32, M=64, W=2, N=97, B=2), 102, "squared"),
    "d64_m32_f32": ("125m", dict(B=2, H=3, N=130, M=32, io="f32"), 103, "squared"),
    "d128_m64_f32": ("1p3b", dict(B=1, H=2, N=150, io="f32"), 104, "squared"),
    "d128_w1_f32": ("1p3b", dict(B=1, H=2, N=70, W=1, io="f32"), 105, "squared"),
    "d64_w8_f32": ("125m", dict(B=1, H=2, N=90, W=8, io="f32"), 106, "squared"),
    "d128_m16_unit_f32": ("1p3b", dict(B=2, H=1, N=100, M=16, io="f32"), 107, "unit"),
    "d64_bf16": ("125m", dict(B=2, H=2, N=130), 108, "squared"),
    "d128_bf16_unit": ("1p3b", dict(B=1, H=2, N=150), 109, "unit"),
}


@pytest.mark.parametrize("name", sorted(BWD))
@pytest.mark.parametrize("mode", ["no_state", "grad_state_only", "state_and_grad_state"])
def test_backward_small(fs, name, mode):
    """Without a state entering, the kernels carry the states divided by bbar
    and form the bbar gradient from per-token totals; the grad_state_only case
    checks that path's state_out terms."""
    from oracle import idattn_backward as OB
    base, over, tag, fn = BWD[name]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    io = s["io"]
    go, gS = _grad_inputs(s, seed=tag)
    with_state = mode == "state_and_grad_state"
    g_S = None if mode == "no_state" else gS
    st0 = tl0 = None
    if with_state:
        st0, tl0 = WL.make_decode_state(s, seed=2)
    want = OB.backward(c.q, c.k, c.v, c.params, go, state_in=st0, tail_in=tl0, grad_state=g_S, feature_norm=fn)
    p = fs.params_to_device(c.params)
    got = fs.backward(up(c.q, io), up(c.k, io), up(c.v, io), p, up(go, io),
                      state_in=None if st0 is None else state_dev(st0), tail_in=None if tl0 is None else up(tl0, io),
                      grad_state=None if g_S is None else state_dev(g_S), feature_norm=fn)
    _sync()
    if not with_state:
        want["state"] = np.zeros((s["B"], s["H"], s["M"], 2 * s["d"]), np.complex128)
        # the gradient of the zero initial state is still defined; compare it
        # with the oracle's by running it from an explicit zero state
        want["state"] = OB.backward(c.q, c.k, c.v, c.params, go, state_in=want["state"], grad_state=g_S,
                                    feature_norm=fn)["state"]
    print(f"backward {name} {mode}", flush=True)
    _compare(f"{name} {mode}", got, want, io, c.params)


@pytest.mark.parametrize("mode", ["no_state", "grad_state_only", "state_and_grad_state"])
def test_backward_zero_and_tiny_bbar(fs, mode):
    """Modes with B = 0 (bbar = 0 exactly) and with B so small that |bbar|
    falls below the bound under which the adjoint scans carry A itself
    rather than conj(bbar) A, next to ordinary modes of the same waves."""
    from oracle import idattn_backward as OB
    base, over, tag, fn = BWD["d64_w8_f32"]
    c = WL.make_case(base, seed=3, tag=tag, **over)
    s = c.spec
    c.params["Bc"][:, 0::5] = 0.0
    c.params["Bc"][:, 2::7] *= 1e-14
    go, gS = _grad_inputs(s, seed=tag + 50)
    with_state = mode == "state_and_grad_state"
    g_S = None if mode == "no_state" else gS
    st0 = tl0 = None
    if with_state:
        st0, tl0 = WL.make_decode_state(s, seed=4)
    zero = np.zeros((s["B"], s["H"], s["M"], 2 * s["d"]), np.complex128)
    want = OB.backward(c.q, c.k, c.v, c.params, go, state_in=zero if st0 is None else st0, tail_in=tl0,
                       grad_state=g_S, feature_norm=fn)
    p = fs.params_to_device(c.params)
    got = fs.backward(up(c.q, "f32"), up(c.k, "f32"), up(c.v, "f32"), p, up(go, "f32"),
                      state_in=None if st0 is None else state_dev(st0), tail_in=None if tl0 is None else up(tl0, "f32"),
                      grad_state=None if g_S is None else state_dev(g_S), feature_norm=fn)
    _sync()
    print(f"backward zero/tiny bbar {mode}", flush=True)
    _compare(f"zero/tiny bbar {mode}", got, want, "f32", c.params)


def test_backward_deterministic_and_zero_tokens(fs):
    """Repeated calls give the same bits; N = 0 gives zero parameter
    gradients and passes grad_state through to grad_state_in."""
    import torch
    base, over, tag, fn = BWD["d64_bf16"]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    go, gS = _grad_inputs(s, seed=5)
    p = fs.params_to_device(c.params)
    args = (up(c.q, "bf16"), up(c.k, "bf16"), up(c.v, "bf16"), p, up(go, "bf16"))
    a = fs.backward(*args, grad_state=state_dev(gS))
    b = fs.backward(*args, grad_state=state_dev(gS))
    _sync()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    B, H, d, M, W = s["B"], s["H"], s["d"], s["M"], s["W"]
    dims = fs.make_dims(B, 0, H, d, M, W, "bf16")
    grads = {key: torch.full_like(p[key], 3.0) for key in PARAM_KEYS}
    gsi = torch.full((B, H, M, 2 * d, 2), 3.0, device="cuda")
    gsd = state_dev(gS)
    fs.idattn_backward(dims, fs.make_params(p), None, None, None, None, None, None, gsd, None, None, None,
                       fs.make_param_grads(grads), gsi, None, 0)
    _sync()
    assert torch.equal(gsi, gsd)
    for key in PARAM_KEYS:
        assert not grads[key].any(), key


@pytest.mark.parametrize("with_state", [True, False], ids=["state_and_grad_state", "no_state"])
def test_backward_full_1p3b_one_head(fs, with_state):
    """The 1.3B workload (B=4 H=16 N=4096 d=128 M=64, bf16) on the GPU; the
    oracle differentiates head 5 over all four batch rows: the input
    gradients of those pairs, that head's parameter gradients and, with a
    state, its state gradient.  no_state is the call the benchmark times (no
    state, tail or state_out gradient)."""
    from oracle import idattn_backward as OB
    import torch
    s = WL.spec("1p3b", tag=110)
    q, k, v = WL.make_rows(s)
    params = WL.make_params(s)
    go, gS = _grad_inputs(s, seed=111)
    st0, tl0 = WL.make_decode_state(s, seed=112)
    if not with_state:
        st0 = tl0 = gS = None
    p = fs.params_to_device(params)
    print(f"backward 1.3B with_state={with_state}: GPU", flush=True)
    got = fs.backward(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), p, up(go, "bf16"),
                      state_in=None if st0 is None else state_dev(st0), tail_in=None if tl0 is None else up(tl0, "bf16"),
                      grad_state=None if gS is None else state_dev(gS))
    _sync()
    h = 5
    hs = slice(h, h + 1)
    print("backward 1.3B: oracle, head 5", flush=True)
    want = OB.backward(q[:, :, hs], k[:, :, hs], v[:, :, hs], {key: val[hs] for key, val in params.items()},
                       go[:, :, hs], state_in=None if st0 is None else st0[:, hs],
                       tail_in=None if tl0 is None else tl0[:, hs], grad_state=None if gS is None else gS[:, hs])
    sub = {key: got[key][:, :, hs] for key in ("q", "k", "v")}
    sub.update({key: got[key][hs] for key in PARAM_KEYS})
    if with_state:
        sub["state"] = got["state"][:, hs]
    _compare(f"1.3B head 5 with_state={with_state}", sub, want, "bf16", {key: val[hs] for key, val in params.items()})
    del got
    torch.cuda.empty_cache()
