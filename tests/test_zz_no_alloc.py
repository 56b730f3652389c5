"""idattn_forward_noalloc (workspace in the library's own scratch array)
against idattn_forward (caller's workspace) through the C ABI: the same
kernels on the same inputs, so the outputs, states and tails must be equal
bit for bit.  Two calls in a row, the second with a smaller input, then the
full 1.3B workload (the largest shape the scratch array is sized for), an
fp32 call on the sequential path, and a shape whose workspace is too large
(rejected before any HIP call)."""
from __future__ import annotations

import pytest

import workloads as WL
from tests.gpu_util import GATE_BF16, check, down, state_dev, state_np, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fixed_state_ssm_amd as fs
    fs.load_library()
    return fs


def _both(fs, s, io, algo, seed):
    """One call through each entry point on the same inputs, state and tail;
    returns the two (o, state_out, tail_out) triples."""
    import torch
    q, k, v = WL.make_rows(s, seed=seed)
    p = fs.params_to_device(WL.make_params(s, seed=seed))
    st0, tl0 = WL.make_decode_state(s, seed=seed + 1)
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]
    dims = fs.make_dims(B, N, H, d, M, W, io, algo)
    prm = fs.make_params(p)
    Q, K, V = up(q, io), up(k, io), up(v, io)
    si, ti = state_dev(st0), up(tl0, io)
    out = []
    for noalloc in (True, False):
        o = torch.empty_like(Q)
        so = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device="cuda")
        to = torch.empty((B, H, 2, W - 1, d), dtype=Q.dtype, device="cuda")
        if noalloc:
            fs.idattn_forward_noalloc(dims, prm, Q, K, V, o, si, ti, so, to)
        else:
            nb = fs.idattn_forward_workspace_size(dims)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            fs.idattn_forward(dims, prm, Q, K, V, o, si, ti, so, to, ws, nb)
        torch.cuda.synchronize()
        out.append((o, so, to))
    return out, (q, k, v, st0, tl0)


def _same(a, b):
    import torch
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_noalloc_matches_forward_two_calls(fs):
    """A call, then a smaller one on the same scratch array."""
    for name, s in (("B4 H16 N700 d128", WL.spec("1p3b", B=4, H=16, N=700, tag=91)),
                    ("B2 H3 N150 d64", WL.spec("125m", B=2, H=3, N=150, tag=92))):
        print(f"noalloc vs forward: {name}", flush=True)
        (a, b), _ = _both(fs, s, "bf16", "chunked", seed=3)
        _same(a, b)


def test_noalloc_full_1p3b_shape(fs):
    """B=4 H=16 N=4096 d=128, the benchmark's workload (161 MiB of scratch):
    bitwise equal to idattn_forward, whose parity the other tests establish."""
    s = WL.spec("1p3b", tag=93)
    nb = fs.idattn_forward_workspace_size(fs.make_dims(4, 4096, 16, 128, 64, 4, "bf16", "chunked"))
    assert nb <= fs.NOALLOC_SCRATCH_BYTES, nb
    print(f"noalloc vs forward: 1.3B shape, {nb} bytes of scratch", flush=True)
    (a, b), _ = _both(fs, s, "bf16", "chunked", seed=5)
    _same(a, b)


def test_noalloc_sequential_f32_against_oracle(fs):
    """The fp32 sequential path through the scratch array, equal to
    idattn_forward and within the fp32 gate of the oracle."""
    import oracle
    s = WL.spec("1p3b", B=2, H=2, N=130, io="f32", tag=94)
    print("noalloc vs forward: f32 sequential", flush=True)
    (a, b), (q, k, v, st0, tl0) = _both(fs, s, "f32", "sequential", seed=7)
    _same(a, b)
    o_ref, st_ref, _ = oracle.forward(q, k, v, WL.make_params(s, seed=7), state_in=st0, tail_in=tl0)
    check("noalloc f32 o", down(a[0]), o_ref, 1e-5, "f32")
    check("noalloc f32 state", state_np(a[1]), st_ref, 1e-5, "f32")


def test_noalloc_bf16_against_oracle(fs):
    import oracle
    s = WL.spec("125m", B=2, H=2, N=333, tag=95)
    (a, _), (q, k, v, st0, tl0) = _both(fs, s, "bf16", "auto", seed=9)
    o_ref, st_ref, _ = oracle.forward(q, k, v, WL.make_params(s, seed=9), state_in=st0, tail_in=tl0)
    check("noalloc bf16 o", down(a[0]), o_ref, GATE_BF16, "bf16")
    check("noalloc bf16 state", state_np(a[1]), st_ref, GATE_BF16, "bf16")


def test_noalloc_rejects_too_large(fs):
    """A workspace beyond the scratch array is an argument error."""
    dims = fs.make_dims(64, 4096, 16, 128, 64, 4, "bf16", "chunked")
    assert fs.idattn_forward_workspace_size(dims) > fs.NOALLOC_SCRATCH_BYTES
    with pytest.raises(fs.IdattnError) as ei:
        fs.idattn_forward_noalloc(dims, fs.make_params({k: 0x10000000 for k in fs.PARAM_KEYS}),
                                  0x20000000, 0x30000000, 0x40000000, 0x50000000)
    assert ei.value.status_name == "IDATTN_ERR_WORKSPACE"
