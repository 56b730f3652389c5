"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments before making any HIP call
(all failing calls below return from validation; no kernel is launched)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import fixed_state_ssm_amd as fs
from fixed_state_ssm_amd.binding import IdattnDims, IdattnParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idattn.h")

FAKE = 0x10000000  # an address that validation never dereferences


def header_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(idattn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_entry_point():
    lib = fs.load_library()
    names = header_entry_points()
    assert set(names) == set(fs.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fs.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (idattn_\w+)$", out, re.M))
    assert set(names) <= exported


def test_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "idattn.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(idattn_dims), offsetof(idattn_dims, io_dtype),
             offsetof(idattn_dims, eps_norm), offsetof(idattn_dims, feature_norm), sizeof(idattn_params),
             offsetof(idattn_params, log_dt), offsetof(idattn_params, Bc), offsetof(idattn_params, rff_omega));
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "t.c")
        exe = os.path.join(td, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    want = [ctypes.sizeof(IdattnDims), IdattnDims.io_dtype.offset, IdattnDims.eps_norm.offset,
            IdattnDims.feature_norm.offset, ctypes.sizeof(IdattnParams), IdattnParams.log_dt.offset,
            IdattnParams.Bc.offset, IdattnParams.rff_omega.offset]
    assert got == want


def test_status_strings_and_version():
    for code, name in fs.STATUS.items():
        assert fs.idattn_status_string(code) == name
    assert fs.idattn_status_string(99) == "IDATTN_ERR_UNKNOWN"
    assert fs.idattn_version() >= 100


def dims(**kw):
    base = dict(B=2, N=64, H=3, d=64, M=32, W=4, io="bf16", algo="auto")
    base.update(kw)
    return fs.make_dims(**base)


PKEYS = ("conv_q", "conv_k", "gain", "bias", "log_dt", "A", "Bc", "rff_omega")


def params(**kw):
    vals = {k: FAKE + 0x1000000 * (i + 1) for i, k in enumerate(PKEYS)}
    vals.update(kw)
    return IdattnParams(*(vals[k] for k in PKEYS))


QB = 0x200000000  # q, k, v, o, ... spaced far apart
ADDR = dict(q=QB, k=2 * QB, v=3 * QB, o=4 * QB, si=5 * QB, ti=6 * QB, so=7 * QB, to=8 * QB, ws=9 * QB)


def call_forward(d, p, ws_bytes=None, **over):
    a = dict(ADDR)
    a.update(over)
    if ws_bytes is None:
        try:
            ws_bytes = fs.idattn_forward_workspace_size(d)
        except fs.IdattnError:
            ws_bytes = 0
    lib = fs.load_library()
    return lib.idattn_forward(ctypes.byref(d), ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["si"], a["ti"],
                              a["so"], a["to"], a["ws"], ws_bytes, None)


def expect(status, name):
    assert fs.STATUS[status] == name, (fs.STATUS[status], fs.idattn_last_error())


@pytest.mark.parametrize("field,value,name", [
    ("B", 0, "IDATTN_ERR_SHAPE"), ("H", -1, "IDATTN_ERR_SHAPE"), ("N", -5, "IDATTN_ERR_SHAPE"),
    ("W", 0, "IDATTN_ERR_SHAPE"), ("d", 48, "IDATTN_ERR_UNSUPPORTED"), ("d", 256, "IDATTN_ERR_UNSUPPORTED"),
    ("M", 8, "IDATTN_ERR_UNSUPPORTED"), ("M", 128, "IDATTN_ERR_UNSUPPORTED"), ("W", 9, "IDATTN_ERR_UNSUPPORTED"),
    ("io", 7, "IDATTN_ERR_ARG"), ("algo", 9, "IDATTN_ERR_ARG"), ("eps_feat", -1.0, "IDATTN_ERR_ARG"),
    ("eps_norm", float("nan"), "IDATTN_ERR_ARG"), ("eps_norm", float("inf"), "IDATTN_ERR_ARG"),
    ("feature_norm", 3, "IDATTN_ERR_ARG"), ("feature_norm", -1, "IDATTN_ERR_ARG"),
])
def test_forward_rejects_bad_dims(field, value, name):
    d = dims(**{field: value})
    expect(call_forward(d, params(), ws_bytes=1 << 40), name)
    assert fs.idattn_last_error()


def test_forward_rejects_null_pointers():
    lib = fs.load_library()
    d = dims()
    assert fs.STATUS[lib.idattn_forward(None, ctypes.byref(params()), *([None] * 9), 0, None)] == "IDATTN_ERR_NULL"
    expect(call_forward(d, params(A=0)), "IDATTN_ERR_NULL")
    expect(call_forward(d, params(), q=0), "IDATTN_ERR_NULL")
    expect(call_forward(d, params(), o=0), "IDATTN_ERR_NULL")
    expect(call_forward(d, params(), ws=0), "IDATTN_ERR_WORKSPACE")


def test_forward_rejects_small_workspace():
    d = dims()
    need = fs.idattn_forward_workspace_size(d)
    assert need > 0
    expect(call_forward(d, params(), ws_bytes=need - 1), "IDATTN_ERR_WORKSPACE")


def test_chunked_needs_bf16():
    with pytest.raises(fs.IdattnError) as e:
        fs.idattn_forward_workspace_size(dims(io="f32", algo="chunked"))
    assert e.value.status_name == "IDATTN_ERR_UNSUPPORTED"


def test_chunked_offset_limit():
    """The chunked kernels address one (b, h) sequence of bf16 [N][H][d] with
    32-bit byte offsets: N H d 2 < 2^31 is chunked, beyond it only the
    sequential path (chosen by AUTO) runs."""
    H, d = 16, 128
    n_ok = (1 << 31) // (H * d * 2) - 1
    assert fs.idattn_forward_workspace_size(dims(B=1, N=n_ok, H=H, d=d, M=64, algo="chunked")) > 0
    with pytest.raises(fs.IdattnError) as e:
        fs.idattn_forward_workspace_size(dims(B=1, N=n_ok + 1, H=H, d=d, M=64, algo="chunked"))
    assert e.value.status_name == "IDATTN_ERR_UNSUPPORTED"
    auto = fs.idattn_forward_workspace_size(dims(B=1, N=n_ok + 1, H=H, d=d, M=64, algo="auto"))
    seq = fs.idattn_forward_workspace_size(dims(B=1, N=n_ok + 1, H=H, d=d, M=64, algo="sequential"))
    assert auto == seq


def test_workspace_size_zero_tokens():
    assert fs.idattn_forward_workspace_size(dims(N=0)) == 0


@pytest.mark.parametrize("over,name", [
    (dict(o=ADDR["q"] + 64), "IDATTN_ERR_ALIAS"),               # o overlaps q
    (dict(so=ADDR["si"] + 16), "IDATTN_ERR_ALIAS"),              # partial state overlap
    (dict(to=ADDR["ti"] + 16), "IDATTN_ERR_ALIAS"),              # partial tail overlap
    (dict(ws=ADDR["v"]), "IDATTN_ERR_ALIAS"),                   # workspace over v
    (dict(so=ADDR["o"]), "IDATTN_ERR_ALIAS"),                   # state_out over o
    (dict(o=FAKE + 0x3000000), "IDATTN_ERR_ALIAS"),             # o over a parameter
    (dict(q=ADDR["q"] + 2), "IDATTN_ERR_ARG"),                  # misaligned
])
def test_forward_rejects_aliasing(over, name):
    expect(call_forward(dims(), params(), **over), name)


def test_decode_validation():
    lib = fs.load_library()
    p = params()

    def dec(d, **over):
        a = dict(q=QB, k=2 * QB, v=3 * QB, o=4 * QB, s=5 * QB, t=6 * QB)
        a.update(over)
        return lib.idattn_decode_step(ctypes.byref(d), ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["s"], a["t"], None)

    expect(dec(dims(N=0)), "IDATTN_ERR_SHAPE")
    expect(dec(dims(N=9)), "IDATTN_ERR_UNSUPPORTED")          # 1..8 tokens per call
    expect(dec(dims(N=4), o=QB + 4 * 2 * 3 * 64 * 2 - 16), "IDATTN_ERR_ALIAS")  # o_t over the end of q_t
    expect(dec(dims(N=1), s=0), "IDATTN_ERR_NULL")
    expect(dec(dims(N=1), t=0), "IDATTN_ERR_NULL")
    expect(dec(dims(N=1), o=QB + 16), "IDATTN_ERR_ALIAS")
    expect(dec(dims(N=1), s=5 * QB + 4), "IDATTN_ERR_ARG")
    expect(dec(dims(N=1, d=100)), "IDATTN_ERR_UNSUPPORTED")


def test_rff_feature_map_validation():
    """The RFF map needs its frequencies; on the chunked path (which AUTO takes
    for bf16 where it has a kernel) its workspace adds the fp16 features of
    queries and keys, B N H d halves each; its frequency table counts as a
    parameter for the overlap checks.  Without the flag the table is not
    looked at: a NULL rff_omega passes on to the next check (here a short
    workspace)."""
    d = dims(feature_norm="rff", M=64, d=128)
    expect(call_forward(d, params(rff_omega=0)), "IDATTN_ERR_NULL")
    expect(call_forward(dims(M=64, d=128), params(rff_omega=0), ws_bytes=1), "IDATTN_ERR_WORKSPACE")
    chunked = fs.idattn_forward_workspace_size(dims(feature_norm="rff", M=64, d=128, algo="chunked"))
    assert chunked == fs.idattn_forward_workspace_size(dims(M=64, d=128, algo="chunked")) + 2 * 2 * 64 * 3 * 128 * 2
    assert fs.idattn_forward_workspace_size(d) == chunked
    assert fs.idattn_forward_workspace_size(dims(feature_norm="rff", M=64, d=128, io="f32")) == \
        fs.idattn_forward_workspace_size(dims(feature_norm="rff", M=64, d=128, algo="sequential", io="f32"))
    with pytest.raises(fs.IdattnError) as e:  # packed batches with it have no chunked kernel
        fs.idattn_forward_varlen_workspace_size(dims(feature_norm="rff", M=64, d=128, algo="chunked"))
    assert e.value.status_name == "IDATTN_ERR_UNSUPPORTED"
    om = params().rff_omega
    table = 3 * 128 * 64 * 4  # H d (d/2) floats
    expect(call_forward(d, params(), o=om + table - 16), "IDATTN_ERR_ALIAS")   # o over the table's end
    expect(call_forward(d, params(), so=om), "IDATTN_ERR_ALIAS")               # state_out over the table


def test_decode_outputs_must_not_overlap_parameters():
    lib = fs.load_library()
    p = params()
    d = dims(N=1, feature_norm="rff", M=64, d=128)
    a = dict(q=QB, k=2 * QB, v=3 * QB, o=4 * QB, s=5 * QB, t=6 * QB)
    for key, where in (("o", p.gain), ("s", p.rff_omega), ("t", p.A)):
        b = dict(a)
        b[key] = where
        expect(lib.idattn_decode_step(ctypes.byref(d), ctypes.byref(p), b["q"], b["k"], b["v"], b["o"], b["s"],
                                      b["t"], None), "IDATTN_ERR_ALIAS")


def call_varlen(d, p, cu, ws_bytes=None, **over):
    a = dict(ADDR)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fs.idattn_forward_varlen_workspace_size(d)
    lib = fs.load_library()
    host = over.get("host")
    return lib.idattn_forward_varlen(ctypes.byref(d), ctypes.byref(p), cu, host, a["q"], a["k"], a["v"], a["o"],
                                     a["si"], a["ti"], a["so"], a["to"], a["ws"], ws_bytes, None)


def test_varlen_validation():
    """Packed batches: B sequences on N = T tokens.  The workspace is that of
    one dense sequence of T tokens; the chunked algorithm is refused; the
    cu_seqlens table must be given, 4-byte aligned and clear of the outputs."""
    d = dims(B=5, N=1000)
    assert fs.idattn_forward_varlen_workspace_size(d) == fs.idattn_forward_workspace_size(
        dims(B=1, N=1000, algo="sequential"))
    assert fs.idattn_forward_varlen_workspace_size(dims(B=5, N=0)) == 0
    with pytest.raises(fs.IdattnError) as e:
        fs.idattn_forward_varlen_workspace_size(dims(B=5, N=1000, algo="chunked"))
    assert e.value.status_name == "IDATTN_ERR_UNSUPPORTED"
    cu = 10 * QB
    p = params()
    expect(call_varlen(d, p, None), "IDATTN_ERR_NULL")
    expect(call_varlen(d, p, cu + 2), "IDATTN_ERR_ARG")
    expect(call_varlen(dims(B=5, N=1000, algo="chunked"), p, cu, ws_bytes=1 << 40), "IDATTN_ERR_UNSUPPORTED")
    expect(call_varlen(dims(B=5, N=1 << 31), p, cu, ws_bytes=1 << 50), "IDATTN_ERR_SHAPE")
    expect(call_varlen(d, p, cu, ws_bytes=fs.idattn_forward_varlen_workspace_size(d) - 1), "IDATTN_ERR_WORKSPACE")
    expect(call_varlen(d, p, cu, o=cu - 64), "IDATTN_ERR_ALIAS")          # o runs into cu_seqlens
    expect(call_varlen(d, p, cu, so=cu - 16), "IDATTN_ERR_ALIAS")         # state_out runs over cu_seqlens
    expect(call_varlen(d, p, cu, o=ADDR["q"] + 1000 * 3 * 64 * 2 - 16), "IDATTN_ERR_ALIAS")  # o over q's last row
    expect(call_varlen(d, p, cu, q=0), "IDATTN_ERR_NULL")
    expect(call_varlen(dims(B=5, N=1000, feature_norm="rff"), params(rff_omega=0), cu), "IDATTN_ERR_NULL")


def test_varlen_chunked_validation():
    """Shapes with a chunked kernel run the packed batch chunked (its plan is
    built on the device, so the device table is required and a host copy is
    optional); a host copy, when given, is checked on the host."""
    d = dims(B=3, N=1000, M=64, d=128)
    cu = 10 * QB
    p = params()
    ok = (ctypes.c_int32 * 4)(0, 10, 10, 1000)
    chunked = fs.idattn_forward_varlen_workspace_size(dims(B=3, N=1000, M=64, d=128, algo="chunked"))
    seq = fs.idattn_forward_varlen_workspace_size(dims(B=3, N=1000, M=64, d=128, algo="sequential"))
    assert fs.idattn_forward_varlen_workspace_size(d) == max(chunked, seq)
    for bad in ((1, 10, 10, 1000), (0, 10, 5, 1000), (0, 10, 10, 999)):
        expect(call_varlen(d, p, cu, host=(ctypes.c_int32 * 4)(*bad)), "IDATTN_ERR_SHAPE")
    dc = dims(B=3, N=1000, M=64, d=128, algo="chunked")
    expect(call_varlen(dc, p, cu, ws_bytes=chunked - 1), "IDATTN_ERR_WORKSPACE")          # no host copy needed
    expect(call_varlen(dc, p, cu, ws_bytes=chunked - 1, host=ok), "IDATTN_ERR_WORKSPACE")
    expect(call_varlen(dims(B=3, N=1000, M=32, d=128, algo="chunked"), p, cu, ws_bytes=1 << 40, host=ok),
           "IDATTN_ERR_UNSUPPORTED")                                        # no kernel for M = 32
    expect(call_varlen(d, p, None, host=ok, ws_bytes=1 << 40), "IDATTN_ERR_NULL")  # the device table is required


def call_normalized(d, p, ws_bytes=None, ei=11 * QB, eo=12 * QB, **over):
    a = dict(ADDR)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fs.idattn_forward_normalized_workspace_size(d)
    lib = fs.load_library()
    return lib.idattn_forward_normalized(ctypes.byref(d), ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["si"],
                                         a["ti"], ei, a["so"], a["to"], eo, a["ws"], ws_bytes, None)


def test_normalized_validation():
    """The normalised readout: a workspace larger than the plain sequential one
    by the denominator shares; the chunked algorithm where the plain readout
    has one (M = 64 here, not M = 32); eta buffers aligned and clear of every
    other buffer (eta_out == eta_in exactly is allowed)."""
    d = dims(algo="sequential")
    plain = fs.idattn_forward_workspace_size(d)
    need = fs.idattn_forward_normalized_workspace_size(d)
    assert need >= plain + 2 * 64 * 3 * 32 * 4
    with pytest.raises(fs.IdattnError) as e:
        fs.idattn_forward_normalized_workspace_size(dims(algo="chunked"))
    assert e.value.status_name == "IDATTN_ERR_UNSUPPORTED"
    p = params()
    expect(call_normalized(d, p, ws_bytes=need - 1), "IDATTN_ERR_WORKSPACE")
    expect(call_normalized(d, p, ei=11 * QB + 8), "IDATTN_ERR_ARG")
    expect(call_normalized(d, p, eo=ADDR["o"] + 32), "IDATTN_ERR_ALIAS")        # eta_out over o
    expect(call_normalized(d, p, eo=11 * QB + 16), "IDATTN_ERR_ALIAS")          # partial overlap with eta_in
    expect(call_normalized(d, p, ei=ADDR["so"]), "IDATTN_ERR_ALIAS")            # state_out over eta_in
    expect(call_normalized(d, p, eo=p.A), "IDATTN_ERR_ALIAS")                   # eta_out over a parameter
    expect(call_normalized(dims(algo="chunked"), p, ws_bytes=1 << 40), "IDATTN_ERR_UNSUPPORTED")
    chunked = fs.idattn_forward_normalized_workspace_size(dims(M=64, algo="chunked"))
    assert chunked == fs.idattn_forward_workspace_size(dims(M=64, algo="chunked"))
    assert fs.idattn_forward_normalized_workspace_size(dims(M=64)) == chunked  # AUTO picks it


def test_decode_normalized_validation():
    lib = fs.load_library()
    p = params()
    d = dims(N=2)

    def dec(**over):
        a = dict(q=QB, k=2 * QB, v=3 * QB, o=4 * QB, s=5 * QB, t=6 * QB, e=11 * QB)
        a.update(over)
        return lib.idattn_decode_step_normalized(ctypes.byref(d), ctypes.byref(p), a["q"], a["k"], a["v"], a["o"],
                                                 a["s"], a["t"], a["e"], None)

    expect(dec(e=None), "IDATTN_ERR_NULL")
    expect(dec(e=11 * QB + 8), "IDATTN_ERR_ARG")
    expect(dec(e=5 * QB + 64), "IDATTN_ERR_ALIAS")   # eta inside the state
    expect(dec(o=11 * QB), "IDATTN_ERR_ALIAS")       # o_t over eta
    expect(dec(e=p.Bc), "IDATTN_ERR_ALIAS")          # eta over a parameter


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    from fixed_state_ssm_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    missing = str(tmp_path / "libidattn.so")
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library(missing)
    monkeypatch.setattr(binding, "LIB_PATH", missing)
    monkeypatch.setattr(binding.load_library, "__defaults__", (missing,))
    with pytest.raises(RuntimeError, match="missing"):
        binding.idattn_version()
    with pytest.raises(RuntimeError, match="missing"):
        binding.idattn_forward_workspace_size(dims())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [1, 2, 3, 8, 16, 40])
def test_varlen_workspace_covers_the_plan(H, d):
    """The packed batch's chunked workspace is sized from B, H and T alone;
    the plan the device builds from the lengths (tests/plan_model.py) must
    fit it for every length mix: at most 256 + B H blocks (the grid), fewer
    than 256 end states, at most min(T, (T + 63 B) / 64) chunks per head, a
    carry list within its capacity.  The workspace also never shrinks as T
    or B grows."""
    import numpy as np

    from tests import plan_model as PM
    rng = np.random.default_rng(H * 1000 + d)
    state = 64 * 2 * d * 2 * 4
    prev_t = {}
    for trial in range(300):
        B = int(rng.choice([1, 2, 3, 8, 40, 300]))
        kind = trial % 3
        if kind == 0:
            lens = rng.integers(0, 3000, size=B)
        elif kind == 1:  # one long sequence among short or empty ones
            lens = rng.integers(0, 70, size=B)
            lens[rng.integers(B)] = int(rng.integers(1000, 40000))
        else:
            lens = rng.geometric(1 / 500, size=B) - 1
        lens = [int(x) for x in lens]
        T = sum(lens)
        if T == 0 or T * H * d * 2 >= 1 << 31:  # the kernels' 32-bit offsets
            continue
        pl = PM.plan(lens, H)
        assert pl["blocks"] <= PM.blocks_max(B, H), (lens, H)
        assert pl["end_states"] < PM.END_STATES, (lens, H)
        assert pl["chunk_slots"] <= H * min(T, (T + 63 * B) // 64), (lens, H)
        assert len(pl["carry"]) <= PM.carry_cap(H), (lens, H)
        assert sorted(b for b, h, seg, c in pl["work"] if seg == pl["S"][b] - 1) == sorted(
            b for b in range(B) for _ in range(H))
        ws = fs.idattn_forward_varlen_workspace_size(fs.make_dims(B, T, H, d, 64, 4, "bf16", "chunked"))
        # the plan-dependent parts alone: plan ints, end states, key-feature tiles
        assert ws >= PM.plan_ints(B, H) * 4 + PM.END_STATES * state + pl["chunk_slots"] * 64 * d * 2
        prev_t.setdefault(B, []).append((T, ws))
    for B, pts in prev_t.items():
        pts.sort()
        assert all(b[1] >= a[1] for a, b in zip(pts, pts[1:])), B
    sizes = [fs.idattn_forward_varlen_workspace_size(fs.make_dims(B, 5000, H, d, 64, 4, "bf16", "chunked"))
             for B in (1, 2, 5, 17, 100)]
    assert sizes == sorted(sizes)


@pytest.mark.parametrize("d", [64, 128])
def test_dense_chunked_plan_matches_model(d):
    """The chunked forward's time split of a dense batch (segment count S and
    size C chunks, chosen by the library's makespan model) equals the plan
    model's, read through the workspace size: with c = 1 chunk the workspace
    is a fixed part plus one tile per (b, h); otherwise it adds S - 1 end
    states and S C tiles per (b, h).  Also the makespan the model minimises,
    for the 125M, 1.3B and 14K shapes: 26 x 3, 16 x 4 and 14 x 16."""
    from tests import plan_model as PM
    state = 64 * 2 * d * 2 * 4
    tile = 64 * d * 2
    for B, H, N in [(8, 12, 4096), (4, 16, 4096), (1, 16, 14336), (8, 16, 700), (8, 12, 700), (4, 16, 200),
                    (1, 2, 1000), (3, 5, 3000), (2, 1, 64 * 37 + 5), (16, 16, 2048), (64, 16, 512)]:
        P = B * H
        ws1 = fs.idattn_forward_workspace_size(fs.make_dims(B, 64, H, d, 64, 4, "bf16", "chunked"))
        fixed = ws1 - P * tile
        S, C = PM.dense_plan(B, H, N)
        ws = fs.idattn_forward_workspace_size(fs.make_dims(B, N, H, d, 64, 4, "bf16", "chunked"))
        assert ws == fixed + (S - 1) * P * state + P * S * C * tile, (B, H, N, S, C)
    assert PM.dense_plan(8, 12, 4096) == (3, 26)
    assert PM.dense_plan(4, 16, 4096) == (4, 16)
    assert PM.dense_plan(1, 16, 14336) == (16, 14)


def test_noalloc_validation():
    """idattn_forward_noalloc rejects, before any HIP call, dims whose
    workspace exceeds the scratch array, and the usual argument errors."""
    lib = fs.load_library()
    prm = fs.make_params({k: FAKE for k in fs.PARAM_KEYS})
    big = fs.make_dims(64, 4096, 16, 128, 64, 4, "bf16", "chunked")
    assert fs.idattn_forward_workspace_size(big) > fs.NOALLOC_SCRATCH_BYTES
    st = lib.idattn_forward_noalloc(ctypes.byref(big), ctypes.byref(prm), FAKE, FAKE + (1 << 32),
                                    FAKE + (2 << 32), FAKE + (3 << 32), None, None, None, None, None)
    assert fs.STATUS[st] == "IDATTN_ERR_WORKSPACE"
    assert "IDATTN_NOALLOC_SCRATCH_BYTES" in fs.idattn_last_error()
    ok = fs.make_dims(4, 4096, 16, 128, 64, 4, "bf16", "chunked")
    assert fs.idattn_forward_workspace_size(ok) <= fs.NOALLOC_SCRATCH_BYTES
    st = lib.idattn_forward_noalloc(ctypes.byref(ok), ctypes.byref(prm), None, FAKE, FAKE, FAKE, None, None,
                                    None, None, None)
    assert fs.STATUS[st] == "IDATTN_ERR_NULL"
    # o overlaps q
    st = lib.idattn_forward_noalloc(ctypes.byref(ok), ctypes.byref(prm), FAKE, FAKE + (1 << 32), FAKE + (2 << 32),
                                    FAKE + 4096, None, None, None, None, None)
    assert fs.STATUS[st] == "IDATTN_ERR_ALIAS"
    text = open(HEADER).read()
    assert "#define IDATTN_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)" in text
    assert fs.NOALLOC_SCRATCH_BYTES == 192 << 20


def test_backward_struct_and_validation():
    """idattn_param_grads matches its C layout; idattn_backward rejects bad
    arguments before any HIP call."""
    from fixed_state_ssm_amd.binding import IdattnParamGrads
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "idattn.h"
    int main(void) {
      printf("%zu %zu %zu\n", sizeof(idattn_param_grads), offsetof(idattn_param_grads, log_dt),
             offsetof(idattn_param_grads, Bc));
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "t.c")
        exe = os.path.join(td, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    assert got == [ctypes.sizeof(IdattnParamGrads), IdattnParamGrads.log_dt.offset, IdattnParamGrads.Bc.offset]

    lib = fs.load_library()
    prm = fs.make_params({k: FAKE for k in fs.PARAM_KEYS})
    g = IdattnParamGrads(*[FAKE + (i + 10 << 32) for i in range(7)])
    dims = fs.make_dims(2, 64, 3, 64, 32, 4, "f32")
    need = fs.idattn_backward_workspace_size(dims)
    assert need > 0

    def call(d=dims, gp=g, ws_bytes=None, **kw):
        a = dict(q=FAKE + (1 << 32), k=FAKE + (2 << 32), v=FAKE + (3 << 32), si=None, ti=None, go=FAKE + (4 << 32),
                 gs=None, gq=FAKE + (5 << 32), gk=FAKE + (6 << 32), gv=FAKE + (7 << 32), gsi=None, ws=FAKE + (8 << 32))
        a.update(kw)
        return fs.STATUS[lib.idattn_backward(ctypes.byref(d), ctypes.byref(prm), a["q"], a["k"], a["v"], a["si"],
                                             a["ti"], a["go"], a["gs"], a["gq"], a["gk"], a["gv"],
                                             ctypes.byref(gp) if gp is not None else None, a["gsi"], a["ws"],
                                             need if ws_bytes is None else ws_bytes, None)]

    assert call(gp=None) == "IDATTN_ERR_NULL"
    assert call(gp=IdattnParamGrads(FAKE + (10 << 32), None, FAKE, FAKE, FAKE, FAKE, FAKE)) == "IDATTN_ERR_NULL"
    assert call(go=None) == "IDATTN_ERR_NULL"
    assert call(ws_bytes=need - 1) == "IDATTN_ERR_WORKSPACE"
    assert call(gq=FAKE + (1 << 32) + 256) == "IDATTN_ERR_ALIAS"          # grad_q overlaps q
    assert call(gk=FAKE + (5 << 32) + 256) == "IDATTN_ERR_ALIAS"          # grad_k overlaps grad_q
    assert call(gsi=FAKE + (8 << 32)) == "IDATTN_ERR_ALIAS"               # grad_state_in overlaps workspace
    assert call(gq=FAKE + (5 << 32) + 8) == "IDATTN_ERR_ARG"              # misaligned
    assert call(d=fs.make_dims(2, 64, 3, 64, 32, 4, "f32", feature_norm="rff")) == "IDATTN_ERR_UNSUPPORTED"
    assert call(d=fs.make_dims(2, 64, 3, 64, 64, 4, "bf16", "chunked")) == "IDATTN_ERR_UNSUPPORTED"
    with pytest.raises(fs.IdattnError):
        fs.idattn_backward_workspace_size(fs.make_dims(2, 64, 3, 64, 32, 4, "f32", feature_norm="rff"))
    assert fs.idattn_backward_workspace_size(fs.make_dims(2, 0, 3, 64, 32, 4, "f32")) == 0
