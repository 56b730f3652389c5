"""The fp64 oracle against its pins (CPU only), and planted mistakes that the
pins must catch."""
import numpy as np
import pytest

from oracle import idattn_oracle as O
from tests.oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn(O)
    assert err <= tol, f"pin {name}: error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- mutations
def _conv_reversed(x, w, hist):
    return _orig["short_conv"](x, np.asarray(w)[..., ::-1], hist)


def _conv_shift(x, w, hist):
    # uses x(i - W + j): every tap one token too far in the past
    x = np.asarray(x, float)
    hist = np.asarray(hist, float)                       # [B, H, W-1, d]
    Wm1 = hist.shape[2]
    full = np.concatenate([hist.transpose(0, 2, 1, 3), x], axis=1)
    full = np.concatenate([np.zeros_like(full[:, :1]), full[:, :-1]], axis=1)
    return _orig["short_conv"](full[:, Wm1:], w, full[:, :Wm1].transpose(0, 2, 1, 3))


def _silu_sign(c):
    c = np.asarray(c, float)
    with np.errstate(over="ignore"):
        return c / (1.0 + np.exp(c))


def _featmap_unsquared(c, eps):
    y = O.silu(c)
    return y / (np.sqrt((y * y).sum(-1, keepdims=True)) + eps)


def _featmap_unit_no_sqrt(c, eps):
    y = O.silu(c)
    return y / ((y * y).sum(-1, keepdims=True) + eps)


def _rff_sin_negated(c, omega):
    xi = _orig["feature_map_rff"](c, omega)
    D = np.asarray(omega).shape[-1]
    return np.concatenate([xi[..., :D], -xi[..., D:]], axis=-1)


def _rff_halves_swapped(c, omega):
    xi = _orig["feature_map_rff"](c, omega)
    D = np.asarray(omega).shape[-1]
    return np.concatenate([xi[..., D:], xi[..., :D]], axis=-1)


def _rff_of_silu(c, omega):
    return _orig["feature_map_rff"](O.silu(c), omega)


def _rff_unscaled(c, omega):
    return _orig["feature_map_rff"](c, omega) * np.sqrt(np.asarray(omega).shape[-1])


def _rff_half_frequency(c, omega):
    return _orig["feature_map_rff"](c, 0.5 * np.asarray(omega))


def _varlen_first_tail(q, k, v, cu, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None,
                       feature_norm="squared"):
    # every sequence takes sequence 0's conv history
    if tail_in is not None:
        tail_in = np.repeat(np.asarray(tail_in)[:1], len(cu) - 1, axis=0)
    return _orig["forward_varlen"](q, k, v, cu, params, eps_feat, eps_norm, state_in, tail_in, feature_norm)


def _varlen_conv_leaks(q, k, v, cu, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None,
                       feature_norm="squared"):
    # the conv of each sequence reads the raw tokens before it in the packed batch
    q, k = np.asarray(q, float), np.asarray(k, float)
    W = params["conv_q"].shape[-1]
    tail = None if tail_in is None else np.array(tail_in, float)
    for b in range(1, len(cu) - 1):
        for j in range(W - 1):
            t = cu[b] - (W - 1) + j
            if t >= 0 and tail is not None:
                tail[b, :, 0, j] = q[t]
                tail[b, :, 1, j] = k[t]
    return _orig["forward_varlen"](q, k, v, cu, params, eps_feat, eps_norm, state_in, tail, feature_norm)


def _eta_without_bbar(q, k, v, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None, eta_in=None,
                      feature_norm="squared", parts=False):
    # the normaliser driven by ones without the input coefficient
    p = dict(params)
    o, st, tl, eta, pt = _orig["forward_normalized"](q, k, v, p, eps_feat, eps_norm, state_in, tail_in, eta_in,
                                                     feature_norm, True)
    num, den = pt["num"], pt["den"]
    abar, bbar = O.zoh(p["log_dt"], p["A"], p["Bc"])
    _, _, _, it = O.forward(q, k, v, p, eps_feat, eps_norm, state_in, tail_in, True, feature_norm)
    e = np.zeros_like(eta) if eta_in is None else np.asarray(eta_in, complex).copy()
    den2 = np.empty_like(den)
    for i in range(den.shape[1]):
        e = abar[None] * e + 1.0
        den2[:, i] = np.einsum("bhm,bhm->bh", it["s"][:, i], e).real
    o2 = num / den2[..., None]
    return (o2, st, tl, e, dict(pt, den=den2)) if parts else (o2, st, tl, e)


def _eta_conjugated(q, k, v, params, eps_feat=1e-6, eps_norm=1e-6, state_in=None, tail_in=None, eta_in=None,
                    feature_norm="squared", parts=False):
    o, st, tl, eta, pt = _orig["forward_normalized"](q, k, v, params, eps_feat, eps_norm, state_in, tail_in,
                                                     eta_in, feature_norm, True)
    num, den = pt["num"], pt["den"]
    abar, bbar = O.zoh(params["log_dt"], params["A"], params["Bc"])
    _, _, _, it = O.forward(q, k, v, params, eps_feat, eps_norm, state_in, tail_in, True, feature_norm)
    e = np.zeros_like(eta) if eta_in is None else np.asarray(eta_in, complex).copy()
    den2 = np.empty_like(den)
    for i in range(den.shape[1]):
        e = abar[None] * e + bbar[None]
        den2[:, i] = np.einsum("bhm,bhm->bh", np.conj(it["s"][:, i]), e).real
    o2 = num / den2[..., None]
    return (o2, st, tl, e, dict(pt, den=den2)) if parts else (o2, st, tl, e)


def _rms_sum(x, g, b, eps):
    x = np.asarray(x, float)
    return np.asarray(g)[None, None] * x / np.sqrt((x * x).sum(-1, keepdims=True) + eps) + np.asarray(b)[None, None]


def _rms_no_bias(x, g, b, eps):
    return _orig["rms_norm"](x, g, np.zeros_like(np.asarray(b, float)), eps)


def _zoh_euler(log_dt, A, Bc):
    abar, _ = _orig["zoh"](log_dt, A, Bc)
    dt = np.exp(np.asarray(log_dt, float))[:, None]
    return abar, dt * (np.asarray(Bc, float)[..., 0] + 1j * np.asarray(Bc, float)[..., 1])


def _zoh_no_dt(log_dt, A, Bc):
    return _orig["zoh"](np.zeros_like(np.asarray(log_dt, float)), A, Bc)


def _step_read_before_update(U, G, xq, zk, zv, a, b):
    s = np.einsum("bhr,bhmr->bhm", xq, U)
    o = np.einsum("bhm,bhmc->bhc", s, G).real
    U = a * U + b * zk[:, :, None, :]
    G = a * G + b * zv[:, :, None, :]
    return U, G, s, o


def _step_conj(U, G, xq, zk, zv, a, b):
    U, G, s, _ = _orig["ssm_step"](U, G, xq, zk, zv, a, b)
    return U, G, s, np.einsum("bhm,bhmc->bhc", np.conj(s), G).real


def _step_swapped_inputs(U, G, xq, zk, zv, a, b):
    return _orig["ssm_step"](U, G, xq, zv, zk, a, b)


def _step_no_bbar_value(U, G, xq, zk, zv, a, b):
    U = a * U + b * zk[:, :, None, :]
    G = a * G + zv[:, :, None, :]
    s = np.einsum("bhr,bhmr->bhm", xq, U)
    return U, G, s, np.einsum("bhm,bhmc->bhc", s, G).real


def _step_imag_dropped(U, G, xq, zk, zv, a, b):
    U, G, s, _ = _orig["ssm_step"](U, G, xq, zk, zv, a, b)
    return U, G, s, np.einsum("bhm,bhmc->bhc", s.real, G.real)


_orig = {name: getattr(O, name) for name in ("short_conv", "silu", "feature_map", "feature_map_unit", "feature_map_rff",
                                             "rms_norm", "forward_varlen", "forward_normalized",
                                             "zoh", "ssm_step")}

MUTANTS = {
    "conv_reversed_taps": ("short_conv", _conv_reversed),
    "conv_off_by_one": ("short_conv", _conv_shift),
    "silu_wrong_sign": ("silu", _silu_sign),
    "featmap_unsquared_norm": ("feature_map", _featmap_unsquared),
    "featmap_unit_without_sqrt": ("feature_map_unit", _featmap_unit_no_sqrt),
    "rff_sin_negated": ("feature_map_rff", _rff_sin_negated),
    "rff_halves_swapped": ("feature_map_rff", _rff_halves_swapped),
    "rff_of_silu": ("feature_map_rff", _rff_of_silu),
    "rff_unscaled": ("feature_map_rff", _rff_unscaled),
    "rff_half_frequency": ("feature_map_rff", _rff_half_frequency),
    "varlen_first_tail_for_all": ("forward_varlen", _varlen_first_tail),
    "varlen_conv_crosses_sequences": ("forward_varlen", _varlen_conv_leaks),
    "eta_driven_without_bbar": ("forward_normalized", _eta_without_bbar),
    "eta_conjugated_scores": ("forward_normalized", _eta_conjugated),
    "rms_sum_not_mean": ("rms_norm", _rms_sum),
    "rms_dropped_bias": ("rms_norm", _rms_no_bias),
    "zoh_euler_bbar": ("zoh", _zoh_euler),
    "zoh_missing_delta": ("zoh", _zoh_no_dt),
    "readout_before_update": ("ssm_step", _step_read_before_update),
    "conjugated_readout": ("ssm_step", _step_conj),
    "key_value_inputs_swapped": ("ssm_step", _step_swapped_inputs),
    "value_bbar_dropped": ("ssm_step", _step_no_bbar_value),
    "imaginary_parts_dropped": ("ssm_step", _step_imag_dropped),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for name, (pin, tol) in PINS.items():
        try:
            err = pin(O)
        except Exception:  # a crash also counts as caught
            err = np.inf
        if not err <= max(tol, 1e-300) * 10:
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"
