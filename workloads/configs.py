"""Named workloads and seeded draws for the Interdomain Attention mixer.

The pages (arXiv 2605.24330 and its two gist.science summaries) train language
models on FineWeb-Edu and print no throughput workload.  The stand-in here is
post-projection activations: q, k, v ~ N(0, 1), i.i.d. over batch rows,
positions, heads and channels, at the head shapes of a 125M-like and a
1.3B-like model at the 4K training context, at 3.5x that context, and at one
decode step after a 2048-token prefill.  Parameters follow the S4D-Lin
initialisation: lambda_m = -0.5 + i*pi*m, B_m = 1, Delta log-uniform on
[1e-3, 1e-1] per head, depthwise conv weights N(0, 1/4) (variance), RMSNorm
gain 1 and bias N(0, 0.02) (standard deviation).

Every draw comes from its own numpy PCG64 stream keyed by
SeedSequence([seed, tag, kind, row]) so that any subset of batch rows can be
regenerated without drawing the others.  kind 0 = parameters, 1 = the q, k, v
of one batch row (drawn in that order, each [N, H, d]), 2 = the decode token
of one row, 3 = a synthetic decode state of one row.

bf16 workloads store float32 draws rounded to bfloat16 with round-to-nearest-
even; the arrays returned here hold those exact bf16 values as float32, and
bf16_bits() gives the 16-bit patterns that a device buffer holds.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

# name -> sizes.  R == d (the short conv is depthwise and the feature map has
# no projection).  W is the short-conv width.
CONFIGS = {
    "tiny":   dict(tag=0, B=1, H=2, N=256, d=16, M=16, W=4, io="f32"),
    "125m":   dict(tag=1, B=8, H=12, N=4096, d=64, M=64, W=4, io="bf16"),
    "1p3b":   dict(tag=2, B=4, H=16, N=4096, d=128, M=64, W=4, io="bf16"),
    "14k":    dict(tag=3, B=1, H=16, N=14336, d=128, M=64, W=4, io="bf16"),
    # decode: B sequences prefilled with N tokens, then one new token each.
    "decode": dict(tag=4, B=256, H=16, N=2048, d=128, M=64, W=4, io="bf16"),
}

KIND_PARAMS, KIND_ROW, KIND_DECODE_TOKEN, KIND_DECODE_STATE, KIND_RFF = 0, 1, 2, 3, 4


def spec(name_or_spec, **overrides) -> dict:
    """Return a config dict (copy), optionally with sizes overridden."""
    if isinstance(name_or_spec, str):
        s = dict(CONFIGS[name_or_spec])
        s["name"] = name_or_spec
    else:
        s = dict(name_or_spec)
        s.setdefault("name", "custom")
    s.update(overrides)
    for key in ("tag", "B", "H", "N", "d", "M", "W"):
        s[key] = int(s[key])
    if s["io"] not in ("f32", "bf16"):
        raise ValueError(f"io must be 'f32' or 'bf16', got {s['io']!r}")
    return s


def _rng(seed: int, tag: int, kind: int, row: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, kind, row])))


# ---------------------------------------------------------------- bf16 storage
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # for every non-NaN pattern u + 0x7FFF + 1 stays below 2**32
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


def _round_bf16_inplace(x: np.ndarray, block: int = 1 << 18) -> None:
    """Round a contiguous float32 array to bfloat16 values in place, in
    cache-sized blocks (same rounding as bf16_bits)."""
    flat = x.reshape(-1)
    u_all = flat.view(np.uint32)
    nan = np.isnan(flat)
    for i in range(0, u_all.size, block):
        u = u_all[i:i + block]
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        u += t
        u &= np.uint32(0xFFFF0000)
    if nan.any():
        u_all[nan] = np.uint32(0x7FC00000)


def _store(x: np.ndarray, io: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if io == "bf16":
        _round_bf16_inplace(x)
    return x


# ---------------------------------------------------------------- parameters
def make_params(s: dict, seed: int = 0) -> dict:
    """Per-head parameters, all float32.

    conv_q, conv_k : [H, d, W]   tap W-1 multiplies the current token
    gain, bias     : [H, 2d]     key-feature half first, then value half
    log_dt         : [H]
    A, Bc          : [H, M, 2]   complex (re, im); A = lambda with Re < 0
    """
    H, d, M, W = s["H"], s["d"], s["M"], s["W"]
    g = _rng(seed, s["tag"], KIND_PARAMS)
    conv_q = g.normal(0.0, 0.5, size=(H, d, W)).astype(np.float32)
    conv_k = g.normal(0.0, 0.5, size=(H, d, W)).astype(np.float32)
    log_dt = g.uniform(math.log(1e-3), math.log(1e-1), size=(H,)).astype(np.float32)
    bias = g.normal(0.0, 0.02, size=(H, 2 * d)).astype(np.float32)
    gain = np.ones((H, 2 * d), dtype=np.float32)
    A = np.zeros((H, M, 2), dtype=np.float32)
    A[:, :, 0] = -0.5
    A[:, :, 1] = (np.pi * np.arange(M, dtype=np.float64)).astype(np.float32)[None, :]
    Bc = np.zeros((H, M, 2), dtype=np.float32)
    Bc[:, :, 0] = 1.0
    return dict(conv_q=conv_q, conv_k=conv_k, gain=gain, bias=bias,
                log_dt=log_dt, A=A, Bc=Bc)


def make_rff_omega(s: dict, seed: int = 0, sigma: float | None = None) -> np.ndarray:
    """Frequencies for the random-Fourier-feature map, float32 [H, d, d/2]:
    i.i.d. N(0, 1/sigma^2) entries (the spectral density of a Gaussian kernel
    of length scale sigma), sigma = sqrt(d)/2 by default so that with unit
    normal inputs the phases are of order 2."""
    H, d = s["H"], s["d"]
    sigma = math.sqrt(d) / 2 if sigma is None else sigma
    g = _rng(seed, s["tag"], KIND_RFF)
    return (g.standard_normal((H, d, d // 2)) / sigma).astype(np.float32)


# ---------------------------------------------------------------- activations
def make_rows(s: dict, rows=None, seed: int = 0, N: int | None = None):
    """q, k, v for the given batch rows: three float32 arrays [len(rows), N, H, d].

    Values are the stored ones (bf16-exact for bf16 workloads).  N overrides
    the sequence length; since q, k and v of a row share one stream, a
    different N gives a different draw, not a prefix.
    """
    rows = list(range(s["B"])) if rows is None else list(rows)
    n = s["N"] if N is None else int(N)
    H, d = s["H"], s["d"]
    q = np.empty((len(rows), n, H, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def one(i_b):
        i, b = i_b
        g = _rng(seed, s["tag"], KIND_ROW, b)
        for arr in (q, k, v):
            g.standard_normal(out=arr[i], dtype=np.float32)
            if s["io"] == "bf16":
                _round_bf16_inplace(arr[i])

    # rows are independent streams; numpy releases the GIL while drawing
    workers = min(len(rows), os.cpu_count() or 1, 16)
    if workers > 1:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, enumerate(rows)))
    else:
        for item in enumerate(rows):
            one(item)
    return q, k, v


def make_decode_token(s: dict, rows=None, seed: int = 0):
    """One new token per row: q_t, k_t, v_t as float32 arrays [len(rows), H, d]."""
    rows = list(range(s["B"])) if rows is None else list(rows)
    H, d = s["H"], s["d"]
    out = [np.empty((len(rows), H, d), dtype=np.float32) for _ in range(3)]
    for i, b in enumerate(rows):
        g = _rng(seed, s["tag"], KIND_DECODE_TOKEN, b)
        for arr in out:
            arr[i] = _store(g.standard_normal((H, d), dtype=np.float32), s["io"])
    return tuple(out)


def make_decode_state(s: dict, rows=None, seed: int = 0, scale: float = 0.1):
    """A synthetic carried state for decode-only tests.

    state: complex64 [len(rows), H, M, 2d] (first d columns = key state U,
    last d = value state Gamma), entries scale * (N(0,1) + i N(0,1)).
    tail: float32 [len(rows), H, 2, W-1, d] raw pre-conv q then k, N(0,1),
    stored in the workload's dtype.
    """
    rows = list(range(s["B"])) if rows is None else list(rows)
    H, d, M, W = s["H"], s["d"], s["M"], s["W"]
    state = np.empty((len(rows), H, M, 2 * d), dtype=np.complex64)
    tail = np.empty((len(rows), H, 2, max(W - 1, 0), d), dtype=np.float32)
    for i, b in enumerate(rows):
        g = _rng(seed, s["tag"], KIND_DECODE_STATE, b)
        re = g.standard_normal((H, M, 2 * d), dtype=np.float32)
        im = g.standard_normal((H, M, 2 * d), dtype=np.float32)
        state[i] = (scale * re + 1j * (scale * im)).astype(np.complex64)
        tail[i] = _store(g.standard_normal((H, 2, max(W - 1, 0), d), dtype=np.float32), s["io"])
    return state, tail


@dataclasses.dataclass
class Case:
    spec: dict
    params: dict
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    rows: list


def make_case(name_or_spec, rows=None, seed: int = 0, **overrides) -> Case:
    s = spec(name_or_spec, **overrides)
    rows = list(range(s["B"])) if rows is None else list(rows)
    q, k, v = make_rows(s, rows, seed)
    return Case(spec=s, params=make_params(s, seed), q=q, k=k, v=v, rows=rows)
