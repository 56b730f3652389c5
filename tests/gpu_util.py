"""Helpers for the GPU parity tests: upload seeded inputs, run the library,
compare with the oracle."""
from __future__ import annotations

import numpy as np

import workloads as WL

GATE_F32 = 1e-5    # all-fp32 path vs fp64 oracle, relative L2
GATE_BF16 = 2e-3   # bf16 I/O with fp32 state vs fp64 oracle, relative L2


def rel_l2(a, b) -> float:
    """||a - b|| / ||b|| over all elements; complex arrays keep both parts."""
    a = np.asarray(a)
    b = np.asarray(b)
    dt = np.complex128 if (np.iscomplexobj(a) or np.iscomplexobj(b)) else np.float64
    a = a.astype(dt)
    b = b.astype(dt)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def up(x, io, dev="cuda"):
    """float32 array holding stored values -> device tensor in the io dtype."""
    import torch
    if io == "bf16":
        return torch.from_numpy(WL.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def down(t) -> np.ndarray:
    return t.float().cpu().numpy()


def state_np(t) -> np.ndarray:
    """float32 [..., 2] device state -> complex128 array."""
    a = t.cpu().numpy().astype(np.float64)
    return a[..., 0] + 1j * a[..., 1]


def state_dev(z, dev="cuda"):
    import torch
    z = np.asarray(z)
    return torch.from_numpy(np.stack([z.real, z.imag], -1).astype(np.float32)).to(dev)


def gate(io):
    return GATE_BF16 if io == "bf16" else GATE_F32


def rel_l2_pairs(a, b) -> np.ndarray:
    """Relative L2 error per (batch row, head) of [B, N, H, d] outputs (over N
    and d), or of [B, H, ...] states (over the trailing axes): [B, H]."""
    a = np.asarray(a)
    b = np.asarray(b)
    dt = np.complex128 if (np.iscomplexobj(a) or np.iscomplexobj(b)) else np.float64
    a = a.astype(dt)
    b = b.astype(dt)
    if a.ndim == 4 and a.shape == b.shape and not np.iscomplexobj(b):  # [B, N, H, d]
        num = np.sqrt((np.abs(a - b) ** 2).sum(axis=(1, 3)))
        den = np.sqrt((np.abs(b) ** 2).sum(axis=(1, 3)))
    else:  # [B, H, ...]
        axes = tuple(range(2, a.ndim))
        num = np.sqrt((np.abs(a - b) ** 2).sum(axis=axes))
        den = np.sqrt((np.abs(b) ** 2).sum(axis=axes))
    return num / np.maximum(den, 1e-300)


def round_io(x, io):
    """The values x takes once stored in the I/O dtype (float32, then bf16)."""
    x = np.asarray(x, dtype=np.float32)
    return WL.bf16_round(x) if io == "bf16" else x


def check(name, got, want, tol, io="f32", pairs=True):
    """Relative L2 of the whole tensor against tol and, with pairs, of every
    (batch row, head) on its own, so that one wrong low-amplitude head cannot
    hide behind the others.  A pair's gate is its own I/O rounding floor plus
    the compute budget the whole-tensor gate leaves, sqrt(f_pair^2 + tol^2 -
    f_whole^2), which is tol wherever the pair's floor is the typical one and
    follows the floor where a pair has few elements.  Real outputs in bf16
    have a floor of about 1.66e-3; fp32 outputs and states almost none.
    Returns (whole, worst pair)."""
    whole = rel_l2(got, want)
    worst = whole
    if pairs:
        e = rel_l2_pairs(got, want)
        if io == "bf16" and not np.iscomplexobj(want):
            r = round_io(want, io)
            f = rel_l2_pairs(r, want)
            f_whole = rel_l2(r, want)
        else:
            f, f_whole = np.zeros_like(e), 0.0
        g = np.sqrt(f ** 2 + max(tol ** 2 - f_whole ** 2, 0.0))
        worst = float(e.max())
        bad = np.argwhere(e > g)
        print(f"{name}: relL2 {whole:.3e}, worst (b, h) {worst:.3e}, worst/gate {float((e / g).max()):.3f} "
              f"(gate {tol:.0e})", flush=True)
        assert bad.size == 0, (name, [(int(i), int(j), float(e[i, j]), float(g[i, j])) for i, j in bad[:8]])
    else:
        print(f"{name}: relL2 {whole:.3e} (gate {tol:.0e})", flush=True)
    assert whole <= tol, (name, whole)
    return whole, worst


def check_packed(name, got, want, cu, tol, io="f32"):
    """check() for a packed batch [T, H, d]: pairs are (sequence, head);
    empty sequences are skipped."""
    got = np.asarray(got)
    want = np.asarray(want)
    cu = [int(x) for x in cu]
    g = [got[None, cu[b]:cu[b + 1]] for b in range(len(cu) - 1) if cu[b + 1] > cu[b]]
    w = [want[None, cu[b]:cu[b + 1]] for b in range(len(cu) - 1) if cu[b + 1] > cu[b]]
    # pad the sequences to one length with zeros (zeros add nothing to either norm)
    n = max(x.shape[1] for x in g)
    pad = lambda x: np.concatenate([x, np.zeros((1, n - x.shape[1]) + x.shape[2:], x.dtype)], axis=1)
    return check(name, np.concatenate([pad(x) for x in g]), np.concatenate([pad(x) for x in w]), tol, io)


def oracle_forward_pool(q, k, v, params, workers=None, **kw):
    """oracle.forward over all heads, the heads split over a thread pool:
    each thread runs the unchanged oracle on its slice of heads (NumPy
    releases the interpreter lock inside the per-step array operations, and
    the threads share the inputs without copies)."""
    import concurrent.futures
    import os

    import oracle
    from threadpoolctl import threadpool_limits
    H = q.shape[2]
    n = workers or min(16, len(os.sched_getaffinity(0)), H)
    bounds = np.linspace(0, H, n + 1).astype(int)

    def one(h0, h1):
        hp = {key: np.asarray(val)[h0:h1] for key, val in params.items()}
        kwh = dict(kw)
        for key in ("state_in", "tail_in"):
            if kwh.get(key) is not None:
                kwh[key] = np.asarray(kwh[key])[:, h0:h1]
        return oracle.forward(q[:, :, h0:h1], k[:, :, h0:h1], v[:, :, h0:h1], hp, **kwh)

    spans = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(len(spans)) as ex:
        res = list(ex.map(lambda ab: one(*ab), spans))
    o = np.concatenate([r[0] for r in res], axis=2)
    st = np.concatenate([r[1] for r in res], axis=1)
    tl = np.concatenate([r[2] for r in res], axis=1)
    return o, st, tl
