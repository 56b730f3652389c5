"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Gates (relative L2 over the compared outputs): 1e-5 for
all-fp32 I/O on the sequential path, 2e-3 for bf16 I/O with fp32 state, over
the whole tensor and over every (batch row, head) on its own (check())."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as WL
from tests.gpu_util import (GATE_BF16, GATE_F32, check, check_packed, down, gate, oracle_forward_pool, rel_l2, rel_l2_pairs,
                             state_dev, state_np, up)

pytestmark = pytest.mark.gpu


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


def _algos(io):
    return ["sequential", "chunked"] if io == "bf16" else ["sequential"]


def _chunked_available(fs, s):
    try:
        fs.idattn_forward_workspace_size(fs.make_dims(s["B"], max(s["N"], 1), s["H"], s["d"], s["M"], s["W"],
                                                      "bf16", "chunked"))
        return True
    except fs.IdattnError:
        return False


# Small shapes the oracle finishes in seconds: several chunks/tiles and a
# ragged tail in time, every supported d and M, W = 1, 2, 4, 8.
SMALL = {  # name: (base config, overrides, seed tag)
    "tiny_f32": ("tiny", {}, 61),
    "tiny_bf16": ("tiny", dict(io="bf16"), 60),
    "d64_m32_ragged_bf16": ("125m", dict(B=2, H=3, N=300, M=32), 55),
    "d64_m64_ragged_f32": ("125m", dict(B=1, H=2, N=211, io="f32"), 56),
    "d128_m64_ragged_bf16": ("1p3b", dict(B=2, H=2, N=333), 51),
    "d128_m16_f32": ("1p3b", dict(B=1, H=2, N=130, M=16, io="f32"), 50),
    "d32_m16_bf16": ("tiny", dict(d=32, M=16, N=150, H=3, B=2, io="bf16"), 54),
    "d16_m64_w2_f32": ("tiny", dict(d=16, M=64, W=2, N=97), 53),
    "d64_w1_bf16": ("125m", dict(B=1, H=2, N=129, W=1), 57),
    # a conv width of 1 with badly conditioned outputs (fp16-operand error 1.27e-3 before
    # the decay tables were carried as fp16 pairs)
    "d64_w1_hard_bf16": ("125m", dict(B=1, H=2, N=129, W=1), 59),
    "d128_w1_bf16": ("1p3b", dict(B=1, H=2, N=129, W=1), 64),
    "d128_w8_bf16": ("1p3b", dict(B=1, H=1, N=70, W=8), 52),
    # conv widths 2 and 3 on the chunked path (its halo holds three tokens)
    "d128_w2_bf16": ("1p3b", dict(B=2, H=2, N=150, W=2), 65),
    "d64_w3_bf16": ("125m", dict(B=2, H=2, N=170, W=3), 66),
    # 64 (b, h) pairs: four time segments of three chunks, the last one ragged
    "d128_segments_bf16": ("1p3b", dict(B=4, H=16, N=700), 62),
    "d64_segments_bf16": ("125m", dict(B=4, H=16, N=700), 63),
    "n1_bf16": ("1p3b", dict(B=3, H=2, N=1), 58),
    "n2_f32": ("tiny", dict(N=2, B=2), 59),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("with_state", [False, True], ids=["zero_state", "given_state"])
def test_small_forward(fs, name, with_state):
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    io = s["io"]
    st0 = tl0 = None
    if with_state:
        st0, tl0 = WL.make_decode_state(s, seed=2)
    o_ref, st_ref, tl_ref = oracle.forward(c.q, c.k, c.v, c.params, state_in=st0, tail_in=tl0)
    p = fs.params_to_device(c.params)
    for algo in _algos(io):
        if algo == "chunked" and not _chunked_available(fs, s):
            continue
        o, st, tl = fs.forward(up(c.q, io), up(c.k, io), up(c.v, io), p, return_state=True, algo=algo,
                               state_in=None if st0 is None else state_dev(st0),
                               tail_in=None if tl0 is None else up(tl0, io))
        _sync()
        check(f"{name} {algo} state={with_state} o", down(o), o_ref, gate(io), io)
        check(f"{name} {algo} state={with_state} state", state_np(st), st_ref, gate(io), io)
        # the tail is a copy of stored inputs: exact
        assert np.array_equal(down(tl), tl_ref.astype(np.float32)), algo


# The unit-norm feature map (xi = y / sqrt(||y||^2 + eps)) on both paths: the
# all-fp32 sequential path, the chunked path with one and with four time
# segments (carry folded into the forward), and d = 64.
UNIT = ["tiny_f32", "d128_m64_ragged_bf16", "d128_segments_bf16", "d64_m32_ragged_bf16", "d64_w1_bf16"]


@pytest.mark.parametrize("name", UNIT)
def test_small_forward_unit_feature_map(fs, name):
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    io = s["io"]
    st0, tl0 = WL.make_decode_state(s, seed=2)
    o_ref, st_ref, _ = oracle.forward(c.q, c.k, c.v, c.params, state_in=st0, tail_in=tl0, feature_norm="unit")
    p = fs.params_to_device(c.params)
    for algo in _algos(io):
        if algo == "chunked" and not _chunked_available(fs, s):
            continue
        o, st, _ = fs.forward(up(c.q, io), up(c.k, io), up(c.v, io), p, return_state=True, algo=algo,
                              state_in=state_dev(st0), tail_in=up(tl0, io), feature_norm="unit")
        _sync()
        check(f"unit {name} {algo} o", down(o), o_ref, gate(io), io)
        check(f"unit {name} {algo} state", state_np(st), st_ref, gate(io), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_step_unit_feature_map(fs, io):
    base, over, tag = SMALL["d128_m64_ragged_bf16"]
    over = dict(over, io=io)
    c = WL.make_case(base, seed=3, tag=tag, **over)
    s = c.spec
    st0, tl0 = WL.make_decode_state(s, seed=4)
    qt, kt, vt = WL.make_decode_token(s)
    ot_ref, st_ref, tl_ref = oracle.decode_step(qt, kt, vt, st0, tl0, c.params, feature_norm="unit")
    p = fs.params_to_device(c.params)
    st = state_dev(st0)
    tl = up(tl0, io)
    ot = fs.decode_step(up(qt, io), up(kt, io), up(vt, io), p, st, tl, feature_norm="unit")
    _sync()
    check(f"unit decode {io} o", down(ot), ot_ref, gate(io), io)
    check(f"unit decode {io} state", state_np(st), st_ref, gate(io), io)
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


# Random Fourier features (Chinese rendering, section 3.1, eq. 6): the
# sequential path of every d (D = d/2 = 8 .. 64 frequencies) from a given state
# and tail, and under AUTO the chunked path where it has a kernel (bf16, d 64 or
# 128, M = 64, W <= 4: the RFF pre-pass feeds the chunked kernels), including
# the folded carry over four segments.  Phases are of order 2 (up to about 10).
RFF = ["tiny_f32", "d16_m64_w2_f32", "d32_m16_bf16", "d64_m32_ragged_bf16", "d64_m64_ragged_f32",
       "d128_m64_ragged_bf16", "d128_m16_f32", "d128_w8_bf16", "d64_w1_bf16", "d128_w2_bf16", "d64_w3_bf16",
       "d128_segments_bf16", "d64_segments_bf16"]


@pytest.mark.parametrize("name", RFF)
def test_forward_rff_feature_map(fs, name):
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    io = s["io"]
    params = dict(c.params, rff_omega=WL.make_rff_omega(s, seed=5))
    st0, tl0 = WL.make_decode_state(s, seed=2)
    o_ref, st_ref, tl_ref = oracle.forward(c.q, c.k, c.v, params, state_in=st0, tail_in=tl0, feature_norm="rff")
    p = fs.params_to_device(params)
    for algo in ("sequential", "auto"):
        o, st, tl = fs.forward(up(c.q, io), up(c.k, io), up(c.v, io), p, return_state=True, algo=algo,
                               state_in=state_dev(st0), tail_in=up(tl0, io), feature_norm="rff")
        _sync()
        check(f"rff {name} {algo} o", down(o), o_ref, gate(io), io)
        check(f"rff {name} {algo} state", state_np(st), st_ref, gate(io), io)
        assert np.array_equal(down(tl), tl_ref.astype(np.float32))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n_tok", [1, 3])
@pytest.mark.parametrize("name", ["d128_m64_ragged_bf16", "d32_m16_bf16"])
def test_decode_step_rff(fs, io, n_tok, name):
    """One and three tokens per call against the oracle's forward over those
    tokens from the same state and tail (the RFF instances of the decode kernel)."""
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=3, tag=tag, **dict(over, io=io))
    s = c.spec
    params = dict(c.params, rff_omega=WL.make_rff_omega(s, seed=6))
    st0, tl0 = WL.make_decode_state(s, seed=4)
    q, k, v = (x[:, :n_tok] for x in (c.q, c.k, c.v))
    o_ref, st_ref, tl_ref = oracle.forward(q, k, v, params, state_in=st0, tail_in=tl0, feature_norm="rff")
    p = fs.params_to_device(params)
    st = state_dev(st0)
    tl = up(tl0, io)
    ot = fs.decode_step(up(q, io), up(k, io), up(v, io), p, st, tl, feature_norm="rff")
    _sync()
    check(f"rff decode {name} {io} n={n_tok} o", down(ot), o_ref, gate(io), io)
    check(f"rff decode {name} {io} n={n_tok} state", state_np(st), st_ref, gate(io), io)
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


# The normalised readout o = num / den (eta state).  Its denominator sums terms
# of both signs and can pass near zero, so o itself is not compared element by
# element: the gate is the componentwise backward error of the ratio,
#   |o_gpu den - num| / (|num| + |o_gpu| sum_m |s_m eta_m|),
# in relative L2 over all outputs.  It is about the rounding unit when o_gpu is
# the exact ratio of a numerator and denominator each computed with rounding
# errors of that size, and of order one when the denominator or the numerator
# is wrong.
def _eta_backward_error(o_gpu, pt):
    num, den, den_abs = pt["num"], pt["den"][..., None], pt["den_abs"][..., None]
    r = o_gpu * den - num
    scale = np.abs(num) + np.abs(o_gpu) * den_abs
    return float(np.linalg.norm(r) / np.linalg.norm(scale))


# shapes on the sequential path (fp32, M = 32 or 16, d = 16) and on the chunked
# one (bf16, d = 64 or 128, M = 64), with one segment and with four (the folded
# carry), and conv widths 1 and 2
NORMALIZED = ["tiny_f32", "d16_m64_w2_f32", "d64_m32_ragged_bf16", "d128_m64_ragged_bf16", "d128_m16_f32",
              "d128_segments_bf16", "d64_segments_bf16", "d64_w1_bf16", "d128_w2_bf16"]


@pytest.mark.parametrize("name", NORMALIZED)
def test_forward_normalized(fs, name):
    import torch
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=1, tag=tag, **over)
    s = c.spec
    io = s["io"]
    st0, tl0 = WL.make_decode_state(s, seed=2)
    r = np.random.default_rng(5)
    eta0 = 0.1 * (r.standard_normal((s["B"], s["H"], s["M"])) + 1j * r.standard_normal((s["B"], s["H"], s["M"])))
    o_ref, st_ref, tl_ref, eta_ref, pt = oracle.forward_normalized(c.q, c.k, c.v, c.params, state_in=st0,
                                                                   tail_in=tl0, eta_in=eta0, parts=True)
    eta_d = torch.from_numpy(np.stack([eta0.real, eta0.imag], -1).astype(np.float32)).cuda()
    p = fs.params_to_device(c.params)
    for algo in _algos(io):
        if algo == "chunked" and not _chunked_available(fs, s):
            continue
        o, st, tl, eta = fs.forward_normalized(up(c.q, io), up(c.k, io), up(c.v, io), p, state_in=state_dev(st0),
                                               tail_in=up(tl0, io), eta_in=eta_d, return_state=True, algo=algo)
        _sync()
        e_o = _eta_backward_error(down(o).astype(np.float64), pt)
        e_eta = rel_l2(state_np(eta), eta_ref)
        print(f"normalized {name} {algo}: o backward error {e_o:.2e}, eta {e_eta:.2e}, "
              f"den < 0 at {float((pt['den'] < 0).mean()):.3f}", flush=True)
        assert e_o <= gate(io), e_o
        check(f"normalized {name} {algo} state", state_np(st), st_ref, gate(io), io)
        assert e_eta <= GATE_F32, e_eta  # eta is fp32 whatever the I/O type
        assert np.array_equal(down(tl), tl_ref.astype(np.float32))
    # the numerator is the plain readout: the same call through idattn_forward
    o_plain = fs.forward(up(c.q, io), up(c.k, io), up(c.v, io), p, state_in=state_dev(st0), tail_in=up(tl0, io),
                         algo="sequential")
    _sync()
    assert rel_l2(down(o_plain), pt["num"]) <= gate(io)


@pytest.mark.parametrize("shape", [dict(B=4, H=16, N=200), dict(B=1, H=2, N=1000)], ids=["fold", "carry"])
def test_forward_normalized_chunked_in_place(fs, shape):
    """The chunked normalised readout with state, tail and eta updated in
    place (one buffer each for input and output), on the folded-carry plan
    (four segments) and the carry-kernel plan (sixteen)."""
    import torch
    c = WL.make_case("1p3b", seed=4, tag=76, **shape)
    s = c.spec
    st0, tl0 = WL.make_decode_state(s, seed=5)
    r = np.random.default_rng(6)
    eta0 = 0.1 * (r.standard_normal((s["B"], s["H"], s["M"])) + 1j * r.standard_normal((s["B"], s["H"], s["M"])))
    _, st_ref, tl_ref, eta_ref, pt = oracle.forward_normalized(c.q, c.k, c.v, c.params, state_in=st0, tail_in=tl0,
                                                               eta_in=eta0, parts=True)
    p = fs.params_to_device(c.params)
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]
    dims = fs.make_dims(B, N, H, d, M, W, "bf16", "chunked")
    nb = fs.idattn_forward_normalized_workspace_size(dims)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    st, tl = state_dev(st0), up(tl0, "bf16")
    eta = torch.from_numpy(np.stack([eta0.real, eta0.imag], -1).astype(np.float32)).cuda()
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    fs.idattn_forward_normalized(dims, fs.make_params(p), up(c.q, "bf16"), up(c.k, "bf16"), up(c.v, "bf16"), o, st, tl,
                                 eta, st, tl, eta, ws, nb)
    _sync()
    e_o = _eta_backward_error(down(o).astype(np.float64), pt)
    print(f"normalized chunked in place {shape}: o backward error {e_o:.2e}", flush=True)
    assert e_o <= GATE_BF16, e_o
    check(f"normalized chunked in place {shape} state", state_np(st), st_ref, GATE_BF16, "bf16")
    assert rel_l2(state_np(eta), eta_ref) <= GATE_F32
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("feature_norm", ["unit", "rff"])
def test_forward_normalized_feature_maps(fs, feature_norm, io):
    import torch
    base, over, tag = SMALL["d64_m32_ragged_bf16"]
    c = WL.make_case(base, seed=14, tag=tag, **dict(over, io=io))
    s = c.spec
    params = dict(c.params, rff_omega=WL.make_rff_omega(s, seed=15))
    st0, tl0 = WL.make_decode_state(s, seed=16)
    o_ref, st_ref, _, eta_ref, pt = oracle.forward_normalized(c.q, c.k, c.v, params, state_in=st0, tail_in=tl0,
                                                              feature_norm=feature_norm, parts=True)
    o, st, _, eta = fs.forward_normalized(up(c.q, io), up(c.k, io), up(c.v, io), fs.params_to_device(params),
                                          state_in=state_dev(st0), tail_in=up(tl0, io), return_state=True,
                                          feature_norm=feature_norm)
    _sync()
    e_o = _eta_backward_error(down(o).astype(np.float64), pt)
    print(f"normalized {feature_norm} {io}: o backward error {e_o:.2e}", flush=True)
    assert e_o <= gate(io), e_o
    assert rel_l2(state_np(st), st_ref) <= gate(io)
    assert rel_l2(state_np(eta), eta_ref) <= GATE_F32


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n_tok", [1, 3, 8])
@pytest.mark.parametrize("name", ["d128_m64_ragged_bf16", "d32_m16_bf16"])
def test_decode_step_normalized(fs, name, n_tok, io):
    """Decode with the normalised readout against the oracle's normalised
    forward over those tokens from the same state, tail and eta."""
    import torch
    base, over, tag = SMALL[name]
    c = WL.make_case(base, seed=17, tag=tag, **dict(over, io=io))
    s = c.spec
    st0, tl0 = WL.make_decode_state(s, seed=18)
    r = np.random.default_rng(19)
    eta0 = 0.5 * (r.standard_normal((s["B"], s["H"], s["M"])) + 1j * r.standard_normal((s["B"], s["H"], s["M"])))
    q, k, v = (x[:, :n_tok] for x in (c.q, c.k, c.v))
    _, st_ref, tl_ref, eta_ref, pt = oracle.forward_normalized(q, k, v, c.params, state_in=st0, tail_in=tl0,
                                                               eta_in=eta0, parts=True)
    st, tl = state_dev(st0), up(tl0, io)
    eta = torch.from_numpy(np.stack([eta0.real, eta0.imag], -1).astype(np.float32)).cuda()
    ot = fs.decode_step(up(q, io), up(k, io), up(v, io), fs.params_to_device(c.params), st, tl, eta=eta)
    _sync()
    e_o = _eta_backward_error(down(ot).astype(np.float64), pt)
    print(f"normalized decode {name} {io} n={n_tok}: o backward error {e_o:.2e}", flush=True)
    assert e_o <= gate(io), e_o
    assert rel_l2(state_np(st), st_ref) <= gate(io)
    assert rel_l2(state_np(eta), eta_ref) <= GATE_F32
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


def test_forward_normalized_split_and_in_place(fs):
    """Two calls, the second resumed from the first's state, tail and eta
    (updated in place), give the one-call result; N = 0 copies eta through."""
    import torch
    base, over, tag = SMALL["d128_m64_ragged_bf16"]
    c = WL.make_case(base, seed=3, tag=tag, **dict(over, io="f32"))
    s = c.spec
    p = fs.params_to_device(c.params)
    q, k, v = up(c.q, "f32"), up(c.k, "f32"), up(c.v, "f32")
    o_all = fs.forward_normalized(q, k, v, p)
    n1 = 150
    o1, st, tl, eta = fs.forward_normalized(q[:, :n1].contiguous(), k[:, :n1].contiguous(), v[:, :n1].contiguous(),
                                            p, return_state=True)
    dims = fs.make_dims(s["B"], s["N"] - n1, s["H"], s["d"], s["M"], s["W"], "f32", "auto")
    nb = fs.idattn_forward_normalized_workspace_size(dims)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q2, k2, v2 = (x[:, n1:].contiguous() for x in (q, k, v))
    o2 = torch.empty_like(q2)
    fs.idattn_forward_normalized(dims, fs.make_params(p), q2, k2, v2, o2, st, tl, eta, st, tl, eta, ws, nb)
    _sync()
    got = torch.cat([o1, o2], 1).cpu().numpy()
    want = o_all.cpu().numpy()
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max() + 1e-30 or rel_l2(got, want) <= 1e-5
    eta_before = eta.clone()
    dz = fs.make_dims(s["B"], 0, s["H"], s["d"], s["M"], s["W"], "f32", "auto")
    eta_out = torch.empty_like(eta)
    fs.idattn_forward_normalized(dz, fs.make_params(p), None, None, None, None, None, None, eta, None, None, eta_out,
                                 None, 0)
    _sync()
    assert torch.equal(eta_out, eta_before)


# Packed variable-length batches: sequences of mixed lengths, some empty and
# some shorter than the conv history, each from its own state and tail.
VARLEN_LENS = [37, 0, 1, 200, 2, 64, 130, 0, 5]


def _packed_case(name, lens, seed, tag_off=0):
    base, over, tag = SMALL[name]
    T = int(sum(lens))
    c = WL.make_case(base, seed=seed, tag=tag + tag_off, **dict(over, B=1, N=max(T, 1)))
    s = dict(c.spec, B=len(lens))
    st0, tl0 = WL.make_decode_state(s, seed=seed + 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return c, s, cu, c.q[0, :T], c.k[0, :T], c.v[0, :T], st0, tl0


# Shapes the chunked kernels take (bf16, d = 64 or 128, M = 64, W <= 4) run
# the packed batch chunked under AUTO (one launch sequence, plan built on the
# device); the others, and SEQUENTIAL, run the sequential path.
@pytest.mark.parametrize("algo", ["auto", "sequential"])
@pytest.mark.parametrize("name", ["tiny_f32", "d16_m64_w2_f32", "d64_m32_ragged_bf16", "d128_m64_ragged_bf16",
                                  "d128_w8_bf16", "d64_w1_bf16", "d128_w2_bf16", "d64_w3_bf16"])
def test_forward_varlen(fs, name, algo):
    import torch
    c, s, cu, q, k, v, st0, tl0 = _packed_case(name, VARLEN_LENS, seed=7)
    io = s["io"]
    o_ref, st_ref, tl_ref = oracle.forward_varlen(q, k, v, cu, c.params, state_in=st0, tail_in=tl0)
    p = fs.params_to_device(c.params)
    cu_d = torch.from_numpy(cu).cuda()
    o, st, tl = fs.forward_varlen(up(q, io), up(k, io), up(v, io), p, cu_d, state_in=state_dev(st0),
                                  tail_in=up(tl0, io), return_state=True, algo=algo)
    _sync()
    tag = f"varlen {name} {algo} T={int(cu[-1])} B={len(cu) - 1}"
    check_packed(f"{tag} o", down(o), o_ref, cu, gate(io), io)
    check(f"{tag} state", state_np(st), st_ref, gate(io), io)
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))
    # an empty sequence passes its state through unchanged
    for b in np.flatnonzero(np.diff(cu) == 0):
        assert np.array_equal(state_np(st)[b], st0[b].astype(np.complex64))


def _oracle_varlen_pool(q, k, v, cu, params, state_in, tail_in):
    """oracle.forward_varlen with each sequence's heads split over threads
    (the same oracle forward per sequence)."""
    outs = [oracle_forward_pool(q[None, cu[b]:cu[b + 1]], k[None, cu[b]:cu[b + 1]], v[None, cu[b]:cu[b + 1]], params,
                                state_in=None if state_in is None else state_in[b:b + 1],
                                tail_in=None if tail_in is None else tail_in[b:b + 1])
            for b in range(len(cu) - 1)]
    return (np.concatenate([r[0][0] for r in outs]), np.concatenate([r[1] for r in outs]),
            np.concatenate([r[2] for r in outs]))


# Packed batches that reach every branch of the device plan (tests/plan_model.py):
# name: (base, overrides, lengths, seed tag)
PACKED = {
    # H = 2: one-chunk segments; sequences of 32 and 11 segments take the carry kernel
    "carry_h2_d128": ("1p3b", dict(H=2), [2000, 30, 0, 700, 5], 201),
    # H = 16: a sequence of 5 segments (carry kernel) beside one of 3 (folded)
    "carry_fold_h16_d128": ("1p3b", dict(H=16), [600, 300, 100], 202),
    # 40 sequences x 16 heads: more pairs than compute units
    "many_h16_d64": ("125m", dict(H=16), None, 203),
    # 300 sequences: last segments in sequence order (no size sort)
    "b300_h1_d64": ("125m", dict(H=1), None, 204),
    # a long and a one-chunk sequence at the 1.3B head shape
    "lens_961_64_h16_d128": ("1p3b", dict(H=16), [961, 64], 207),
}


def _packed_lens(name):
    base, over, lens, tag = PACKED[name]
    if lens is None:
        r = np.random.default_rng(tag)
        lens = [int(x) for x in r.integers(0, 300, size=40 if name.startswith("many") else 300)]
        lens[3] = 0
    return lens


@pytest.mark.parametrize("name", sorted(PACKED))
def test_forward_varlen_chunked_plans(fs, name):
    """The packed chunked path against the oracle on batches whose plans take
    the carry kernel, the folded carry, more pairs than compute units and
    more sequences than the plan sorts, with state and tail updated in place
    (state_out = state_in, tail_out = tail_in)."""
    import torch
    base, over, _, tag = PACKED[name]
    lens = _packed_lens(name)
    T = int(sum(lens))
    c = WL.make_case(base, seed=1, tag=tag, **dict(over, B=1, N=T))
    s = dict(c.spec, B=len(lens))
    st0, tl0 = WL.make_decode_state(s, seed=tag)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = c.q[0], c.k[0], c.v[0]
    print(f"packed {name}: B={len(lens)} T={T} H={s['H']} d={s['d']}", flush=True)
    p = fs.params_to_device(c.params)
    st, tl = state_dev(st0), up(tl0, "bf16")
    o = fs.forward_varlen_into(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), p, torch.from_numpy(cu).cuda(),
                               state_in=st, tail_in=tl, state_out=st, tail_out=tl, algo="chunked")
    _sync()
    o_ref, st_ref, tl_ref = _oracle_varlen_pool(q, k, v, cu, c.params, st0, tl0)
    check_packed(f"packed {name} o", down(o), o_ref, cu, GATE_BF16, "bf16")
    check(f"packed {name} state", state_np(st), st_ref, GATE_BF16, "bf16")
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


@pytest.mark.parametrize("case", ["varlen_h2", "bench_mix_h16", "many_h16", "b300_h1"])
def test_varlen_device_plan(fs, case):
    """The plan the tables kernel builds from the device table, read back from
    the workspace, equals the plan model's (segment size, block counts, the
    per-sequence offsets, the order of the last segments, the carry list)."""
    import torch

    from tests import plan_model as PM
    lens, H, d = {"varlen_h2": (VARLEN_LENS, 2, 128),
                  "bench_mix_h16": ([6000, 3500, 2500, 2048, 1200, 700, 400, 36], 16, 128),
                  "many_h16": (_packed_lens("many_h16_d64"), 16, 64),
                  "b300_h1": (_packed_lens("b300_h1_d64"), 1, 64)}[case]
    B, T = len(lens), int(sum(lens))
    s = WL.spec("1p3b" if d == 128 else "125m", B=1, N=T, H=H, tag=205)
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    x = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    dims = fs.make_dims(B, T, H, d, 64, 4, "bf16", "chunked")
    nbytes = fs.idattn_forward_varlen_workspace_size(dims)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    fs.idattn_forward_varlen(dims, fs.make_params(p), cu, x, x, x, o, None, None, None, None, ws, nbytes)
    _sync()
    n = PM.plan_ints(B, H)
    got = ws[:4 * n].cpu().view(torch.int32).numpy()
    want = PM.plan_array(lens, H)
    assert list(got[:len(want)]) == want, case


def test_varlen_malformed_table_writes_nothing(fs):
    """A device table that does not rise from 0 to T gives the packed chunked
    path a plan of no blocks: no output, state or tail is written."""
    import torch
    T, H, d = 300, 2, 128
    s = WL.spec("1p3b", B=1, N=T, H=H, tag=206)
    p = fs.params_to_device(WL.make_params(s))
    x = torch.ones((T, H, d), dtype=torch.bfloat16, device="cuda")
    for bad in ([0, 200, 100, 300], [5, 100, 200, 300], [0, 100, 200, 299]):
        o = torch.full_like(x, 7.0)
        st = torch.full((3, H, 64, 2 * d, 2), 7.0, device="cuda")
        tl = torch.full((3, H, 2, 3, d), 7.0, dtype=torch.bfloat16, device="cuda")
        fs.forward_varlen_into(x, x, x, p, torch.tensor(bad, dtype=torch.int32, device="cuda"), o=o,
                               state_out=st, tail_out=tl, algo="chunked")
        _sync()
        assert bool((o == 7).all()) and bool((st == 7).all()) and bool((tl == 7).all()), bad


@pytest.mark.parametrize("feature_norm", ["unit", "rff"])
def test_forward_varlen_feature_maps(fs, feature_norm):
    """Packed batches with the other feature maps (the flag reaches the packed
    path's feature kernel unchanged)."""
    import torch
    c, s, cu, q, k, v, st0, tl0 = _packed_case("d128_m64_ragged_bf16", [70, 0, 3, 150, 1], seed=12)
    params = dict(c.params, rff_omega=WL.make_rff_omega(s, seed=13))
    o_ref, st_ref, tl_ref = oracle.forward_varlen(q, k, v, cu, params, state_in=st0, tail_in=tl0,
                                                  feature_norm=feature_norm)
    o, st, tl = fs.forward_varlen(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), fs.params_to_device(params),
                                  torch.from_numpy(cu).cuda(), state_in=state_dev(st0), tail_in=up(tl0, "bf16"),
                                  return_state=True, feature_norm=feature_norm)
    _sync()
    assert rel_l2(down(o), o_ref) <= GATE_BF16
    assert rel_l2(state_np(st), st_ref) <= GATE_BF16
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


def test_forward_varlen_without_state(fs):
    """No state_in / tail_in: every sequence starts from zeros."""
    import torch
    c, s, cu, q, k, v, _, _ = _packed_case("d64_m32_ragged_bf16", [3, 90, 0, 41], seed=9)
    o_ref, st_ref, tl_ref = oracle.forward_varlen(q, k, v, cu, c.params)
    o, st, tl = fs.forward_varlen(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), fs.params_to_device(c.params),
                                  torch.from_numpy(cu).cuda(), return_state=True)
    _sync()
    assert rel_l2(down(o), o_ref) <= GATE_BF16
    assert rel_l2(state_np(st), st_ref) <= GATE_BF16
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_varlen_sequential_matches_dense_at_scale(fs, io):
    """At the 1.3B head shape (H = 16, d = 128, M = 64) with 9 400 packed tokens:
    every sequence of the packed sequential call gives bit for bit what the
    dense sequential forward gives for that sequence alone (the same kernels
    in the same order; the dense path is itself compared with the oracle)."""
    import torch
    lens = [4096, 1, 3000, 0, 17, 2286]
    s = WL.spec("1p3b", B=1, N=sum(lens), io=io, tag=81)
    q, k, v = WL.make_rows(s, seed=3)
    params = WL.make_params(s, seed=3)
    st0, tl0 = WL.make_decode_state(dict(s, B=len(lens)), seed=4)
    p = fs.params_to_device(params)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qd, kd, vd = up(q[0], io), up(k[0], io), up(v[0], io)
    o, st, tl = fs.forward_varlen(qd, kd, vd, p, torch.from_numpy(cu).cuda(), state_in=state_dev(st0),
                                  tail_in=up(tl0, io), return_state=True, algo="sequential")
    stb, tlb = state_dev(st0), up(tl0, io)
    for b, n in enumerate(lens):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        ob, sb, tb = fs.forward(qd[None, sl], kd[None, sl], vd[None, sl], p, algo="sequential",
                                state_in=stb[b:b + 1], tail_in=tlb[b:b + 1], return_state=True)
        _sync()
        assert torch.equal(o[sl], ob[0]), b
        assert torch.equal(st[b], sb[0]), b
        assert torch.equal(tl[b], tb[0]), b


def test_forward_varlen_chunked_at_scale(fs):
    """The packed batch the benchmark times (1.3B head shape, 8 sequences of
    6000 .. 36 tokens, T = 16 384), from a seeded state and tail, against the
    oracle over every (sequence, head) pair: output, end state and tail."""
    import torch
    lens = [6000, 3500, 2500, 2048, 1200, 700, 400, 36]
    s = WL.spec("1p3b", B=1, N=sum(lens), tag=90)
    q, k, v = WL.make_rows(s)
    params = WL.make_params(s)
    st0, tl0 = WL.make_decode_state(dict(s, B=len(lens)), seed=91)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = fs.params_to_device(params)
    print("packed 1.3B mix: GPU", flush=True)
    o, st, tl = fs.forward_varlen(up(q[0], "bf16"), up(k[0], "bf16"), up(v[0], "bf16"), p,
                                  torch.from_numpy(cu).cuda(), state_in=state_dev(st0), tail_in=up(tl0, "bf16"),
                                  return_state=True, algo="chunked")
    _sync()
    o_np, st_np, tl_np = down(o), state_np(st), down(tl)
    del o, st, tl
    print("packed 1.3B mix: oracle over all (sequence, head) pairs", flush=True)
    o_ref, st_ref, tl_ref = _oracle_varlen_pool(q[0], k[0], v[0], cu, params, st0, tl0)
    check_packed("packed 1.3B mix o", o_np, o_ref, cu, GATE_BF16, "bf16")
    check("packed 1.3B mix state", st_np, st_ref, GATE_BF16, "bf16")
    assert np.array_equal(tl_np, tl_ref.astype(np.float32))


# Learned decays can be much faster than the S4D-Lin init: Delta |Re lambda| up
# to 6 per token.  A ragged last chunk must still leave an exact end state
# (before the fix, a zero-padded chunk corrected by abar^-(L-n) lost the state:
# relative error 2.5e-2 at Delta = 0.1, Re lambda = -2 and NaN at Delta = 1).
# Shapes: six one-chunk segments with the carry kernel (B=1, H=2, N=333), and
# four segments with the carry folded into the forward (B=4, H=16, N=200).
@pytest.mark.parametrize("dt,re_lam", [(0.1, -2.0), (0.3, -2.0), (1.0, -0.5), (3.0, -2.0)])
@pytest.mark.parametrize("shape", [dict(B=1, H=2, N=333), dict(B=4, H=16, N=200, d=64)], ids=["carry", "fold"])
def test_ragged_end_state_fast_decay(fs, dt, re_lam, shape):
    c = WL.make_case("1p3b", seed=1, tag=71, **shape)
    s = c.spec
    p = dict(c.params)
    p["log_dt"] = np.full_like(p["log_dt"], np.log(dt))
    A = np.array(p["A"])
    A[..., 0] = re_lam
    p["A"] = A.astype(np.float32)
    st0, tl0 = WL.make_decode_state(s, seed=2)
    o_ref, st_ref, _ = oracle.forward(c.q, c.k, c.v, p, state_in=st0, tail_in=tl0)
    pd = fs.params_to_device(p)
    o, st, _ = fs.forward(up(c.q, "bf16"), up(c.k, "bf16"), up(c.v, "bf16"), pd, return_state=True, algo="chunked",
                          state_in=state_dev(st0), tail_in=up(tl0, "bf16"))
    _sync()
    check(f"dt={dt} re={re_lam} {shape} o", down(o), o_ref, GATE_BF16, "bf16")
    check(f"dt={dt} re={re_lam} {shape} state", state_np(st), st_ref, GATE_BF16, "bf16")


# Small steps: bbar ~ Delta B down to 1e-8.  The decay table is scaled per head
# by a power of two so that it stays in the fp16 normal range (before, the
# output error was 7.4e-3 at Delta = 1e-3, B = 0.01 and 2.7e-2 at Delta = 1e-6);
# Delta -> 0 is also the limit the oracle is pinned against.
@pytest.mark.parametrize("dt,b_scale", [(1e-3, 0.01), (1e-5, 1.0), (1e-6, 1.0), (1e-6, 0.01), (0.05, 300.0)])
@pytest.mark.parametrize("shape", [dict(B=1, H=2, N=333), dict(B=4, H=16, N=200, d=64)], ids=["carry", "fold"])
def test_small_step_scaled_tables(fs, dt, b_scale, shape):
    c = WL.make_case("1p3b", seed=1, tag=72, **shape)
    s = c.spec
    p = dict(c.params)
    p["log_dt"] = np.full_like(p["log_dt"], np.log(dt))
    Bc = np.array(p["Bc"])
    Bc[..., 0] *= b_scale
    p["Bc"] = Bc.astype(np.float32)
    st0, tl0 = WL.make_decode_state(s, seed=2, scale=0.1 * dt * b_scale)
    o_ref, st_ref, _ = oracle.forward(c.q, c.k, c.v, p, state_in=st0, tail_in=tl0)
    pd = fs.params_to_device(p)
    o, st, _ = fs.forward(up(c.q, "bf16"), up(c.k, "bf16"), up(c.v, "bf16"), pd, return_state=True, algo="chunked",
                          state_in=state_dev(st0), tail_in=up(tl0, "bf16"))
    _sync()
    check(f"dt={dt} B*{b_scale} {shape} o", down(o), o_ref, GATE_BF16, "bf16")
    check(f"dt={dt} B*{b_scale} {shape} state", state_np(st), st_ref, GATE_BF16, "bf16")


# The chunked path holds the queries' SiLU outputs and the mode scores as fp16
# operands; each token's y' is scaled by a power of two and the rest of its
# scale applied on the output, so queries of any scale keep the gate.  q, k
# scaled by exact powers of two (the stored inputs stay bf16); before the
# per-token scaling, 2^-12 and 2^13 gave non-finite outputs.
@pytest.mark.parametrize("feature_norm", ["squared", "unit"])
@pytest.mark.parametrize("e", [-12, -8, -4, 8, 11, 13])
def test_chunked_query_scale_range(fs, e, feature_norm):
    c = WL.make_case("1p3b", seed=1, tag=73, B=1, H=2, N=333)
    sc = 2.0 ** e
    q, k = np.asarray(c.q) * sc, np.asarray(c.k) * sc
    o_ref, st_ref, _ = oracle.forward(q, k, c.v, c.params, feature_norm=feature_norm)
    p = fs.params_to_device(c.params)
    for algo in ("sequential", "chunked"):
        o, st, _ = fs.forward(up(q, "bf16"), up(k, "bf16"), up(c.v, "bf16"), p, return_state=True, algo=algo,
                              feature_norm=feature_norm)
        _sync()
        check(f"q, k x 2^{e} {feature_norm} {algo} o", down(o), o_ref, GATE_BF16, "bf16")
        check(f"q, k x 2^{e} {feature_norm} {algo} state", state_np(st), st_ref, GATE_BF16, "bf16")


# Several tokens per decode call (one sweep of the state for all of them)
# against the oracle's forward over the same tokens from the same state and
# tail: outputs of every token, the new state and the shifted tail.
@pytest.mark.parametrize("n_tok", [2, 3, 8])
@pytest.mark.parametrize("case", ["d128_m64_w4", "d64_m32_w8", "d128_m16_w1_unit"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_multi_token(fs, n_tok, case, io):
    base, over = {"d128_m64_w4": ("1p3b", dict(B=3, H=2)), "d64_m32_w8": ("125m", dict(B=2, H=3, M=32, W=8)),
                  "d128_m16_w1_unit": ("1p3b", dict(B=2, H=2, M=16, W=1))}[case]
    fn = "unit" if case.endswith("unit") else "squared"
    c = WL.make_case(base, seed=5, tag=75, N=n_tok, io=io, **over)
    s = c.spec
    st0, tl0 = WL.make_decode_state(s, seed=6)
    o_ref, st_ref, tl_ref = oracle.forward(c.q, c.k, c.v, c.params, state_in=st0, tail_in=tl0, feature_norm=fn)
    p = fs.params_to_device(c.params)
    st = state_dev(st0)
    tl = up(tl0, io)
    o = fs.decode_step(up(c.q, io), up(c.k, io), up(c.v, io), p, st, tl, feature_norm=fn)
    _sync()
    check(f"decode x{n_tok} {case} {io} o", down(o), o_ref, gate(io), io)
    check(f"decode x{n_tok} {case} {io} state", state_np(st), st_ref, gate(io), io)
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


def _pairs(s, n, seed):
    r = np.random.default_rng(seed)
    idx = r.choice(s["B"] * s["H"], size=min(n, s["B"] * s["H"]), replace=False)
    return sorted((int(i // s["H"]), int(i % s["H"])) for i in idx)


def _head_params(p, h):
    return {k: np.asarray(v)[h:h + 1] for k, v in p.items()}


_FULL = {}  # config -> (GPU o, GPU state, oracle o, oracle state), shared by the tests below


def _full_config(fs, cfg):
    """The whole workload of a config on the GPU (the launch the benchmark
    times) and the oracle over every (b, h) pair (threads over heads)."""
    import torch
    if cfg not in _FULL:
        s = WL.spec(cfg)
        q, k, v = WL.make_rows(s)
        params = WL.make_params(s)
        p = fs.params_to_device(params)
        print(f"{cfg}: GPU forward B={s['B']} H={s['H']} N={s['N']} d={s['d']}", flush=True)
        o, st, _ = fs.forward(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), p, return_state=True)
        _sync()
        o_np, st_np = down(o), state_np(st)
        del o, st
        torch.cuda.empty_cache()
        print(f"{cfg}: oracle over all {s['B'] * s['H']} (b, h) pairs", flush=True)
        o_ref, st_ref, _ = oracle_forward_pool(q, k, v, params)
        _FULL[cfg] = (o_np, st_np, o_ref, st_ref)
    return _FULL[cfg]


@pytest.mark.parametrize("cfg", ["125m", "1p3b", "14k"])
def test_full_config_all_pairs(fs, cfg):
    """Every (b, h) pair of the 125M, 1.3B and 14K workloads, end to end,
    against the oracle: the output and the end state, whole and per pair."""
    o, st, o_ref, st_ref = _full_config(fs, cfg)
    assert np.isfinite(o).all()
    check(f"{cfg} o", o, o_ref, GATE_BF16, "bf16")
    check(f"{cfg} state", st, st_ref, GATE_BF16, "bf16")
    e = rel_l2_pairs(o, o_ref)
    print(f"{cfg}: per-pair o relL2 min {e.min():.3e} median {np.median(e):.3e} max {e.max():.3e}", flush=True)


@pytest.mark.parametrize("variant", ["unit", "rff", "normalized"])
def test_full_shape_variants_sampled_pairs(fs, variant):
    """The feature-map and readout variants at the full 1.3B shape (B=4 H=16
    N=4096 d=128 M=64, bf16 I/O), all on the chunked path (RFF through its
    pre-pass); the oracle recomputes two (b, h) sequences end to end."""
    import torch
    s = WL.spec("1p3b")
    q, k, v = WL.make_rows(s)
    params = WL.make_params(s)
    if variant == "rff":
        params["rff_omega"] = WL.make_rff_omega(s, seed=1)
    p = fs.params_to_device(params)
    qd, kd, vd = up(q, "bf16"), up(k, "bf16"), up(v, "bf16")
    fn = "squared" if variant == "normalized" else variant
    if variant == "normalized":
        o, st, _, eta = fs.forward_normalized(qd, kd, vd, p, return_state=True)
    else:
        o, st, _ = fs.forward(qd, kd, vd, p, return_state=True, feature_norm=fn)
    _sync()
    for b, h in _pairs(s, 2, seed=11):
        args = (q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], _head_params(params, h))
        if variant == "normalized":
            _, st_ref, _, eta_ref, pt = oracle.forward_normalized(*args, parts=True)
            e = _eta_backward_error(down(o[b:b + 1, :, h:h + 1]).astype(np.float64), pt)
            assert rel_l2(state_np(eta[b, h]), eta_ref[0, 0]) <= GATE_F32
        else:
            o_ref, st_ref, _ = oracle.forward(*args, feature_norm=fn)
            e = rel_l2(down(o[b, :, h]), o_ref[0, :, 0])
        e_s = rel_l2(state_np(st[b, h]), st_ref[0, 0])
        print(f"1p3b {variant} pair b={b} h={h}: o error {e:.3e} state relL2 {e_s:.3e}", flush=True)
        assert e <= GATE_BF16 and e_s <= GATE_BF16
    del o, st
    torch.cuda.empty_cache()


def test_length_statistics_14k(fs):
    """At 3.5x the 4K context the per-head rms of o over 1024-token windows
    is flat after warm-up (max/min over [7168, 14336) <= 1.25 for every head)
    and equals the oracle's window statistics."""
    o, _, o_ref, _ = _full_config(fs, "14k")

    def windows(x):
        return np.sqrt((np.asarray(x, np.float64)[0].reshape(14, 1024, 16, 128) ** 2).mean(axis=(1, 3)))

    win, win_ref = windows(o), windows(o_ref)  # [window, head]
    ratio = win[7:].max(0) / win[7:].min(0)
    print("window rms (rows = 1024-token windows, cols = heads):\n", np.array2string(win, precision=4))
    dev = np.abs(win / win_ref - 1.0)
    print(f"window rms vs oracle: max relative difference {dev.max():.2e}", flush=True)
    assert np.isfinite(win).all()
    assert ratio.max() <= 1.25, ratio
    assert (win_ref[7:].max(0) / win_ref[7:].min(0)).max() <= 1.25
    # a window rms is an average over 16 384 outputs, so its relative error is
    # far below the per-element gate
    assert dev.max() <= GATE_BF16, dev.max()


def test_config0_own_seed(fs):
    """The tiny workload exactly as specified (B=1, H=2, N=256, d=R=16,
    M=16, fp32, seed 0) on the all-fp32 path at 1e-5, and in bf16 I/O."""
    c = WL.make_case("tiny")
    o_ref, st_ref, tl_ref = oracle.forward(c.q, c.k, c.v, c.params)
    p = fs.params_to_device(c.params)
    o, st, tl = fs.forward(up(c.q, "f32"), up(c.k, "f32"), up(c.v, "f32"), p, return_state=True)
    _sync()
    check("tiny seed 0 f32 o", down(o), o_ref, GATE_F32, "f32")
    check("tiny seed 0 f32 state", state_np(st), st_ref, GATE_F32, "f32")
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))
    cb = WL.make_case("tiny", io="bf16")
    ob_ref, stb_ref, _ = oracle.forward(cb.q, cb.k, cb.v, cb.params)
    ob, stb, _ = fs.forward(up(cb.q, "bf16"), up(cb.k, "bf16"), up(cb.v, "bf16"), p, return_state=True)
    _sync()
    check("tiny seed 0 bf16 o", down(ob), ob_ref, GATE_BF16, "bf16")
    check("tiny seed 0 bf16 state", state_np(stb), stb_ref, GATE_BF16, "bf16")


def test_decode_step_full_batch(fs):
    """Decode at 256 sequences x 16 heads from a seeded synthetic state and tail;
    every o_t and every updated state entry against the oracle."""
    s = WL.spec("decode")
    st0, tl0 = WL.make_decode_state(s, seed=3)
    qt, kt, vt = WL.make_decode_token(s)
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    st = state_dev(st0)
    tl = up(tl0, "bf16")
    ot = fs.decode_step(up(qt, "bf16"), up(kt, "bf16"), up(vt, "bf16"), p, st, tl)
    _sync()
    ot_ref, st_ref, tl_ref = oracle.decode_step(qt, kt, vt, st0, tl0, params)
    check("decode o_t", down(ot), ot_ref, GATE_BF16, "bf16")
    check("decode state", state_np(st), st_ref, GATE_BF16, "bf16")
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


def test_decode_multi_token_full_batch(fs):
    """Four tokens per decode call at 256 sequences x 16 heads (the call the
    benchmark times) from a seeded synthetic state and tail: every output,
    every updated state entry and the tail against the oracle's forward over
    the same four tokens."""
    s = WL.spec("decode")
    st0, tl0 = WL.make_decode_state(s, seed=8)
    q, k, v = WL.make_rows(s, seed=9, N=4)  # [B, 4, H, d] each
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    st = state_dev(st0)
    tl = up(tl0, "bf16")
    o = fs.decode_step(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), p, st, tl)
    _sync()
    o_ref, st_ref, tl_ref = oracle_forward_pool(q, k, v, params, state_in=st0, tail_in=tl0)
    check("decode x4 o", down(o), o_ref, GATE_BF16, "bf16")
    check("decode x4 state", state_np(st), st_ref, GATE_BF16, "bf16")
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))


def test_decode_step_f32_gate(fs):
    s = WL.spec("1p3b", B=4, io="f32")
    st0, tl0 = WL.make_decode_state(s, seed=4)
    qt, kt, vt = WL.make_decode_token(s)
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    st = state_dev(st0)
    tl = up(tl0, "f32")
    ot = fs.decode_step(up(qt, "f32"), up(kt, "f32"), up(vt, "f32"), p, st, tl)
    _sync()
    ot_ref, st_ref, _ = oracle.decode_step(qt, kt, vt, st0, tl0, params)
    assert rel_l2(down(ot), ot_ref) <= GATE_F32
    assert rel_l2(state_np(st), st_ref) <= GATE_F32


def test_prefill_then_decode(fs):
    """The decode workload end to end: a 2048-token prefill of 256 sequences
    on the GPU returning state and tail, then one decode step.  The step is
    checked on all 256 x 16 (b, h) pairs against the oracle's decode step
    from the same prefilled state and tail (copied back from the GPU); the
    prefill itself on eight seeded sequences, all heads, against the
    oracle's own prefill."""
    import torch
    s = WL.spec("decode")
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    q, k, v = WL.make_rows(s)
    print("decode: GPU prefill of 256 x 2048 tokens", flush=True)
    o, st, tl = fs.forward(up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), p, return_state=True)
    del o
    _sync()
    st_pre, tl_pre = state_np(st), down(tl)
    qt, kt, vt = WL.make_decode_token(s)
    ot = fs.decode_step(up(qt, "bf16"), up(kt, "bf16"), up(vt, "bf16"), p, st, tl)
    _sync()
    print("decode: oracle step from the GPU prefill state", flush=True)
    ot_ref, st2_ref, tl2_ref = oracle.decode_step(qt, kt, vt, st_pre, tl_pre, params)
    check("decode from prefill o_t", down(ot), ot_ref, GATE_BF16, "bf16")
    check("decode from prefill state", state_np(st), st2_ref, GATE_BF16, "bf16")
    assert np.array_equal(down(tl), tl2_ref.astype(np.float32))
    rows = sorted(np.random.default_rng(8).choice(s["B"], size=8, replace=False).tolist())
    print(f"decode: oracle prefill of rows {rows}", flush=True)
    _, st_ref, tl_ref = oracle_forward_pool(q[rows], k[rows], v[rows], params)
    check("prefill state (8 rows)", st_pre[rows], st_ref, GATE_BF16, "bf16")
    assert np.array_equal(tl_pre[rows], tl_ref.astype(np.float32))
    del st, tl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", ["sequential", "chunked"])
def test_split_resume_and_determinism(fs, algo):
    """forward over N tokens equals two calls chained through state and tail
    (any size, no oracle needed), and repeated calls are bitwise equal."""
    s = WL.spec("1p3b", B=2, H=4, N=1000)
    if algo == "chunked" and not _chunked_available(fs, s):
        pytest.skip("chunked path not built")
    q, k, v = WL.make_rows(s, seed=5)
    p = fs.params_to_device(WL.make_params(s))
    Q, K, V = up(q, "bf16"), up(k, "bf16"), up(v, "bf16")
    o1, st1, tl1 = fs.forward(Q, K, V, p, return_state=True, algo=algo)
    o1b = fs.forward(Q, K, V, p, algo=algo)
    _sync()
    assert np.array_equal(down(o1), down(o1b))
    n1 = 389
    oa, sa, ta = fs.forward(Q[:, :n1].contiguous(), K[:, :n1].contiguous(), V[:, :n1].contiguous(), p,
                            return_state=True, algo=algo)
    ob, sb, tb = fs.forward(Q[:, n1:].contiguous(), K[:, n1:].contiguous(), V[:, n1:].contiguous(), p,
                            state_in=sa, tail_in=ta, return_state=True, algo=algo)
    _sync()
    both = np.concatenate([down(oa), down(ob)], axis=1)
    assert rel_l2(both, down(o1)) <= GATE_BF16
    # the chunked path rounds state-update operands to fp16 (about 3e-4 relative
    # state error against the oracle); the sequential path is plain fp32
    assert rel_l2(state_np(sb), state_np(st1)) <= (1e-5 if algo == "sequential" else GATE_BF16)
    assert np.array_equal(down(tb), down(tl1))


def test_in_place_state_and_zero_tokens(fs):
    import torch
    s = WL.spec("125m", B=1, H=2, N=50, io="f32")
    q, k, v = WL.make_rows(s, seed=6)
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    st0, tl0 = WL.make_decode_state(s, seed=6)
    st = state_dev(st0)
    tl = up(tl0, "f32")
    dims = fs.make_dims(1, 50, 2, 64, 64, 4, "f32", "sequential")
    nb = fs.idattn_forward_workspace_size(dims)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o = torch.empty((1, 50, 2, 64), dtype=torch.float32, device="cuda")
    fs.idattn_forward(dims, fs.make_params(p), up(q, "f32"), up(k, "f32"), up(v, "f32"), o, st, tl, st, tl, ws, nb)
    _sync()
    o_ref, st_ref, tl_ref = oracle.forward(q, k, v, params, state_in=st0, tail_in=tl0)
    assert rel_l2(down(o), o_ref) <= GATE_F32
    assert rel_l2(state_np(st), st_ref) <= GATE_F32
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))
    # N = 0: no tokens; state and tail pass through, or become zeros
    d0 = fs.make_dims(1, 0, 2, 64, 64, 4, "f32")
    st2 = torch.full_like(st, 7.0)
    tl2 = torch.full_like(tl, 7.0)
    fs.idattn_forward(d0, fs.make_params(p), None, None, None, None, st, tl, st2, tl2, None, 0)
    _sync()
    assert torch.equal(st2, st) and torch.equal(tl2, tl)
    fs.idattn_forward(d0, fs.make_params(p), None, None, None, None, None, None, st2, tl2, None, 0)
    _sync()
    assert not st2.any() and not tl2.any()


# (B, H, N, d) -> time segments per sequence in the library's plan (modelled in
# tests/plan_model.py): 1 (short, one segment), 2, 3 and 4 (the carry folded
# into the forward, as in the 125M and 1.3B plans; fold_s3_uneven has segments
# of 5, 5 and 1 chunks) and 16 (the carry kernel).
IN_PLACE = {"n2_s1": (1, 2, 2, 128), "n50_s1": (1, 2, 50, 128), "fold_s4_d128": (4, 16, 200, 128),
            "fold_s4_d64": (4, 16, 200, 64), "fold_s3_d128": (4, 16, 150, 128), "fold_s2_d64": (8, 16, 700, 64),
            "fold_s3_uneven_d64": (8, 12, 700, 64), "carry_s16": (1, 2, 1000, 128),
            "carry_s16_h16": (1, 16, 1000, 128)}


@pytest.mark.parametrize("case", sorted(IN_PLACE))
def test_in_place_state_and_tail_chunked(fs, case):
    """The chunked path with state_out = state_in and tail_out = tail_in (the
    same buffers), for every way the plan carries the state into a segment."""
    import torch
    B, H, N, d = IN_PLACE[case]
    s = WL.spec("1p3b" if d == 128 else "125m", B=B, H=H, N=N)
    if not _chunked_available(fs, s):
        pytest.skip("chunked path not built")
    q, k, v = WL.make_rows(s, seed=7)
    params = WL.make_params(s)
    p = fs.params_to_device(params)
    st0, tl0 = WL.make_decode_state(s, seed=7)
    st = state_dev(st0)
    tl = up(tl0, "bf16")
    dims = fs.make_dims(B, N, H, d, 64, 4, "bf16", "chunked")
    nb = fs.idattn_forward_workspace_size(dims)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    print(f"in-place chunked {case}", flush=True)
    fs.idattn_forward(dims, fs.make_params(p), up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), o, st, tl, st, tl, ws, nb)
    _sync()
    o_ref, st_ref, tl_ref = oracle.forward(q, k, v, params, state_in=st0, tail_in=tl0)  # bf16-exact inputs
    check(f"in-place {case} o", down(o), o_ref, GATE_BF16, "bf16")
    check(f"in-place {case} state", state_np(st), st_ref, GATE_BF16, "bf16")
    assert np.array_equal(down(tl), tl_ref.astype(np.float32))
