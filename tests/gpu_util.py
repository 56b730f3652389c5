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
