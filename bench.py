"""Benchmark of the Interdomain Attention mixer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1p3b]

A step is one idattn_forward over the whole workload batch (short conv,
feature map, RMSNorm, ZOH tables, key scan, value scan + readout, state and
tail emission), inputs already resident in HBM.  Three copies of the inputs
are rotated so that consecutive steps do not re-read the previous step's
bytes from the 256 MB last-level cache.  Prints one JSON line.

The roofline object covers the forward launch: algorithmic bytes (read q, k,
v once, write o once: 8 d bytes per token-head in bf16) divided by the mean
duration of a launch: two HIP events on the launch stream around the K timed
launches, divided by K (the gaps between launches included).  Events between
the launches would add a marker to the stream after every call: measured,
they cost about 6 us per step at the 1.3B shape.
Traffic (bytes actually moved, from rocprofv3 FETCH_SIZE / WRITE_SIZE) comes
from the committed profile summary when it was taken on the current kernel
source, else null.

The CPU baseline is the fp64 oracle, single-threaded, on a bounded sample of
the same workload (the first batch rows with every head and whole sequences,
or a prefix of row 0 when one row exceeds the time target).

Before the W warmup steps the forward runs back to back for --settle-s
seconds (0.3 by default), untimed: the GPU's clocks take several dozen
launches to reach their steady state, and without it a short warmup times
that ramp instead of the kernels.  The number of settle launches is reported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mixer tokens/sec fwd (1.3B shape, N=4096) + % of HBM roofline, 1 GPU"
HBM_PEAK_GBPS = 8000.0
FP32_PEAK_TFLOPS = 157.3
FP16_MFMA_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = ["fixed_state_ssm_amd/csrc/chunked_ws.hip", "fixed_state_ssm_amd/csrc/backward.hip",
                  "fixed_state_ssm_amd/csrc/featmap.hip", "fixed_state_ssm_amd/csrc/scan_seq.hip",
                  "fixed_state_ssm_amd/csrc/decode.hip", "fixed_state_ssm_amd/csrc/common.h",
                  "fixed_state_ssm_amd/csrc/launch.h", "fixed_state_ssm_amd/csrc/api.cpp"]


def source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(config: str, algo: str):
    """Bytes per launch from profiles/forward_<algo>__<config>_traffic.md if
    its recorded source hash matches the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"forward_{algo}__{config}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != source_sha():
        return None
    return float(m_b.group(1))


def plan_segments(B, N, H, L=64):
    """The chunked forward's time split of a dense batch, as the library plans
    it: S segments of Lseg tokens per (b, h), the segment size (in chunks)
    with the least modelled makespan on 256 compute units (full segments
    dispatched first, then the shorter last ones; 1.5 chunk times of fixed
    work per workgroup), searched from half to twice the even split."""
    import heapq
    P, c = B * H, (N + L - 1) // L
    if c <= 1:
        return 1, L

    def makespan(C):
        S = -(-c // C)
        loads = [0.0] * 256
        for size in [C] * (P * (S - 1)) + [c - (S - 1) * C] * P:
            heapq.heappush(loads, heapq.heappop(loads) + size + 1.5)
        return max(loads)

    even = -(-P * c // 256)
    lo, hi = max(1, even // 2), min(2 * even, c)
    lo = min(lo, hi)
    step = (hi - lo) // 512 + 1
    best, best_t = c, makespan(c)
    for C in range(hi, lo - 1, -step):
        t = makespan(C)
        if t < best_t - 1e-9:
            best, best_t = C, t
    return -(-c // best), best * L


def chunked_mfma_flops(B, N, H, d, L=64):
    """Flops the chunked forward issues on v_mfma_f32_16x16x32_f16 (16 384
    each) per launch, counted from the kernels' loops, every product with the
    decay table counted twice (its high and low fp16 parts).  Per chunk of one
    (b, h): the forward runs G (10 causal 16x16 tiles, d/32 K steps), Y U^T
    (4 d/32 per key wave, 8 waves), the U update (4 d/16 per key wave), S (16
    per key wave), the P~ tiles (10 x 8), X Gamma (16 per value wave owning
    columns, d/16 of them), the Gamma update (32 each) and P~ Z_v (8 each);
    the feature pass repeats the two state updates for every segment but the
    last of a sequence."""
    S, lseg = plan_segments(B, N, H, L)
    rt, kb, own = d // 16, d // 32, d // 16
    fwd = 10 * kb + 8 * 4 * kb + 8 * 4 * rt + 8 * 16 + 80 + own * (16 + 32 + 8)
    feat = 8 * 4 * rt + own * 32
    chunks_total = B * H * ((N + L - 1) // L)
    chunks_upd = B * H * (S - 1) * (lseg // L)
    return 16384.0 * (fwd * chunks_total + feat * chunks_upd)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks take several dozen back-to-back launches to settle; a short
    # warmup times that ramp (about 15 % slower at the 1.3B shape) instead of the
    # steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="1p3b", choices=["125m", "1p3b", "14k"])
    ap.add_argument("--algo", default="auto", choices=["auto", "sequential", "chunked"])
    ap.add_argument("--feature-norm", default="squared", choices=["squared", "unit", "rff"],
                    help="feature map xi = y / (||y||^2 + eps) (squared), y / sqrt(||y||^2 + eps) (unit), or "
                         "random Fourier features of the conv output (rff; the chunked path then runs an RFF pre-pass)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU sample")
    ap.add_argument("--only", choices=["varlen", "normalized", "rff", "backward", "decode"],
                    help="run one of the secondary measurements alone and print it (for profiling)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed back-to-back forwards before the warmup steps (clock settle)")
    return ap.parse_args()


def cpu_baseline(s, q, k, v, params, target_s: float, feature_norm: str = "squared"):
    """The oracle as it stands, one thread, on a bounded sample: the first
    batch rows (every head), whole sequences when they fit the time target,
    else a prefix of row 0."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(limits=1):
        n0 = 32
        t = time.perf_counter()
        oracle.forward(q[:1, :n0], k[:1, :n0], v[:1, :n0], params, feature_norm=feature_norm)
        per_tok = (time.perf_counter() - t) / n0  # one row, every head
        budget_tok = target_s / max(per_tok, 1e-9)
        rows = int(max(1, min(s["B"], budget_tok // s["N"])))
        n = int(max(n0, min(s["N"], budget_tok)))
        t = time.perf_counter()
        o, _, _ = oracle.forward(q[:rows, :n], k[:rows, :n], v[:rows, :n], params, feature_norm=feature_norm)
        dt = time.perf_counter() - t
    assert np.isfinite(o).all()
    return {"value": rows * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"batch rows 0..{rows - 1}, all {s['H']} heads, first {n} of {s['N']} tokens "
                      f"({dt:.1f} s, fp64 NumPy, 1 thread)"}


def measure_copy_gbps(torch, nbytes=2 << 30):
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def measure_inplace_gbps(torch, nbytes=1090519040):
    """Read + write rate of a plain in-place elementwise pass (torch's mul_)
    over a buffer the size of the decode workload's state: the streaming
    rate that a kernel updating its state in place can hope for."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    a.mul_(1.0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a.mul_(1.0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a
    return 2 * nbytes / (ms * 1e-3) / 1e9


def decode_bench(torch, fs, steps, warmup):
    """Decode workload: 256 sequences x 16 heads, d = R = 128, M = 64, prefilled
    by a 2048-token forward on N(0,1) inputs drawn on the device, then one
    token per sequence per step (state updated in place)."""
    import workloads as WL
    s = WL.spec("decode")
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]
    p = fs.params_to_device(WL.make_params(s))
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    x = [torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]
    _, state, tail = fs.forward(x[0], x[1], x[2], p, return_state=True)
    del x
    tok = [torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]
    o_t = torch.empty_like(tok[0])
    dims = fs.make_dims(B, 1, H, d, M, W, "bf16")
    prm = fs.make_params(p)
    for _ in range(warmup):
        fs.idattn_decode_step(dims, prm, tok[0], tok[1], tok[2], o_t, state, tail)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fs.idattn_decode_step(dims, prm, tok[0], tok[1], tok[2], o_t, state, tail)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    med = ms[len(ms) // 2]
    nbytes = 2 * B * H * M * 2 * d * 8 + 4 * B * H * d * 2 + 2 * B * H * 2 * (W - 1) * d * 2
    # several tokens per sequence in one call: the decode step over NT tokens
    # (one sweep of the state for all of them), state and tail in place
    multi = {}
    for NT in (4, 8):
        tk = [torch.randn((B, NT, H, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]
        o_m = torch.empty_like(tk[0])
        dims_m = fs.make_dims(B, NT, H, d, M, W, "bf16")
        for _ in range(warmup):
            fs.idattn_decode_step(dims_m, prm, tk[0], tk[1], tk[2], o_m, state, tail)
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            fs.idattn_decode_step(dims_m, prm, tk[0], tk[1], tk[2], o_m, state, tail)
            e1.record()
        torch.cuda.synchronize()
        ms_m = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        med_m = ms_m[len(ms_m) // 2]
        multi[f"tokens_{NT}"] = {"ms_per_call_median": med_m, "tokens_per_s": B * NT / (med_m * 1e-3)}
    # the normalised readout: one token per sequence, eta carried in place
    eta = torch.zeros((B, H, M, 2), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        fs.idattn_decode_step_normalized(dims, prm, tok[0], tok[1], tok[2], o_t, state, tail, eta)
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record()
        fs.idattn_decode_step_normalized(dims, prm, tok[0], tok[1], tok[2], o_t, state, tail, eta)
        e1.record()
    torch.cuda.synchronize()
    ms_n = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    med_n = ms_n[len(ms_n) // 2]
    normalized = {"path": "idattn_decode_step_normalized, one token per sequence, eta in place",
                  "ms_per_step_median": med_n, "tokens_per_s": B / (med_n * 1e-3)}
    return {"workload": "decode: 256 sequences x 16 heads, d=R=128, M=64, W=4, bf16 I/O, fp32 state "
                        "prefilled by a 2048-token forward",
            "tokens_per_s": B / (med * 1e-3), "ms_per_step_median": med,
            "multi_token": dict(multi, path="idattn_decode_step with several tokens per sequence, state and tail in place"),
            "normalized": normalized,
            "roofline": {"bound": "hbm", "achieved": nbytes / (med * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "algorithmic_bytes": nbytes}}


def time_calls(torch, call, steps, warmup, settle_s=0.3):
    """Mean time of one call (HIP events on the current stream around the
    timed calls, divided by their number, as for the main forward) after
    settle_s seconds of back-to-back calls and warmup more, the same clock
    settle the main forward measurement gets."""
    t = time.perf_counter()
    while time.perf_counter() - t < settle_s:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def varlen_bench(torch, fs, WL, dense_ms=None, steps=20, warmup=5):
    """Packed variable-length batch at the 1.3B head shape (H=16, d=128, M=64,
    W=4, bf16): 16 384 tokens (the dense 1.3B batch's count) in 8 sequences
    of mixed lengths (long prompts beside short ones).  AUTO runs the chunked
    kernels in one launch sequence whose plan is built on the device from
    the sequence table; the sequential fp32 path is timed beside it.  Each
    call is timed with HIP events on the stream after the same clock settle
    as the dense forward."""
    import numpy as np
    lens = [6000, 3500, 2500, 2048, 1200, 700, 400, 36]
    s = WL.spec("1p3b", B=1, N=sum(lens), tag=90)
    q, k, v = WL.make_rows(s)
    p = fs.params_to_device(WL.make_params(s))
    prm = fs.make_params(p)
    B, T, H, d, M, W = len(lens), sum(lens), s["H"], s["d"], s["M"], s["W"]

    def up(x):
        return torch.from_numpy(WL.bf16_bits(x[0]).view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = up(q), up(k), up(v)
    o = torch.empty_like(qd)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    state = torch.zeros((B, H, M, 2 * d, 2), dtype=torch.float32, device="cuda")
    tail = torch.zeros((B, H, 2, W - 1, d), dtype=torch.bfloat16, device="cuda")

    def timed(algo):
        dims = fs.make_dims(B, T, H, d, M, W, "bf16", algo)
        nbytes = fs.idattn_forward_varlen_workspace_size(dims)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

        def call():
            fs.idattn_forward_varlen(dims, prm, cu, qd, kd, vd, o, None, None, state, tail, ws, nbytes)

        return time_calls(torch, call, steps if algo == "auto" else 3, warmup, 0.3 if algo == "auto" else 0.0)

    ms = timed("auto")
    ms_seq = timed("sequential")
    out = {"workload": f"packed batch: {B} sequences, lengths {lens} (T={T}), H={H} d=R={d} M={M} W={W}, "
                       f"bf16 I/O",
           "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
           "path": "chunked kernels, one launch sequence, plan built on the device from the sequence table",
           "sequential": {"ms_per_call": ms_seq, "tokens_per_s": T / (ms_seq * 1e-3),
                          "path": "sequential fp32 path"}}
    if dense_ms:
        out["dense_1p3b_ms_per_call"] = dense_ms
        out["ratio_to_dense"] = ms / dense_ms
    return out


def normalized_bench(torch, fs, WL, config, plain_ms=None, steps=20, warmup=5):
    """The forward with the normalised readout (eta state) at the bench's
    shape: the chunked path where the plain readout has one (AUTO), with eta
    carried out; also the sequential path for comparison."""
    import numpy as np
    s = WL.spec(config)
    q, k, v = WL.make_rows(s)
    p = fs.params_to_device(WL.make_params(s))
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]

    def up(x):
        return torch.from_numpy(WL.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = up(q), up(k), up(v)
    o = torch.empty_like(qd)
    state = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device="cuda")
    eta = torch.empty((B, H, M, 2), dtype=torch.float32, device="cuda")
    prm = fs.make_params(p)
    out = {}
    for algo in ("auto", "sequential"):
        dims = fs.make_dims(B, N, H, d, M, W, "bf16", algo)
        nbytes = fs.idattn_forward_normalized_workspace_size(dims)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

        def call():
            fs.idattn_forward_normalized(dims, prm, qd, kd, vd, o, None, None, None, state, None, eta, ws, nbytes)

        ms = time_calls(torch, call, steps if algo == "auto" else 3, warmup, 0.3 if algo == "auto" else 0.0)
        out[algo] = {"ms_per_call": ms, "tokens_per_s": B * N / (ms * 1e-3)}
        del ws
    try:
        fs.idattn_forward_normalized_workspace_size(fs.make_dims(B, N, H, d, M, W, "bf16", "chunked"))
        path = "chunked (MFMA) path"
    except fs.IdattnError:
        path = "sequential fp32 path"
    res = {"workload": f"{config}: B={B} H={H} N={N} d=R={d} M={M} W={W}, bf16 I/O, normalised readout (eta), "
                       f"{path}", "ms_per_call": out["auto"]["ms_per_call"],
           "tokens_per_s": out["auto"]["tokens_per_s"],
           "sequential": dict(out["sequential"], path="sequential fp32 path")}
    if plain_ms:
        res["ratio_to_plain_forward"] = out["auto"]["ms_per_call"] / plain_ms
    return res


def rff_bench(torch, fs, WL, config, plain_ms=None, steps=20, warmup=5):
    """The forward with the random-Fourier-feature map (frequencies drawn as
    in the tests) at the bench's shape: AUTO (the chunked path, its RFF
    pre-pass included) and the sequential path for comparison."""
    import numpy as np
    s = WL.spec(config)
    q, k, v = WL.make_rows(s)
    params = WL.make_params(s)
    params["rff_omega"] = WL.make_rff_omega(s, seed=1)
    p = fs.params_to_device(params)
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]

    def up(x):
        return torch.from_numpy(WL.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = up(q), up(k), up(v)
    o = torch.empty_like(qd)
    state = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device="cuda")
    prm = fs.make_params(p)
    out = {}
    for algo in ("auto", "sequential"):
        dims = fs.make_dims(B, N, H, d, M, W, "bf16", algo, feature_norm="rff")
        nbytes = fs.idattn_forward_workspace_size(dims)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

        def call():
            fs.idattn_forward(dims, prm, qd, kd, vd, o, None, None, state, None, ws, nbytes)

        ms = time_calls(torch, call, steps if algo == "auto" else 3, warmup, 0.3 if algo == "auto" else 0.0)
        out[algo] = {"ms_per_call": ms, "tokens_per_s": B * N / (ms * 1e-3)}
        del ws
    try:
        fs.idattn_forward_workspace_size(fs.make_dims(B, N, H, d, M, W, "bf16", "chunked", feature_norm="rff"))
        path = "chunked (MFMA) path with the RFF pre-pass"
    except fs.IdattnError:
        path = "sequential fp32 path"
    res = {"workload": f"{config}: B={B} H={H} N={N} d=R={d} M={M} W={W}, bf16 I/O, random Fourier features "
                       f"(d/2 frequencies per head), {path}", "ms_per_call": out["auto"]["ms_per_call"],
           "tokens_per_s": out["auto"]["tokens_per_s"],
           "sequential": dict(out["sequential"], path="sequential fp32 path")}
    if plain_ms:
        res["ratio_to_plain_forward"] = out["auto"]["ms_per_call"] / plain_ms
    return res


def backward_bench(torch, fs, WL, config, steps=5, warmup=2):
    """idattn_backward at the bench's shape (bf16 I/O, fp32 arithmetic, the
    sequential algorithm): every gradient of a forward over the workload,
    inputs and the output gradient resident in HBM."""
    import numpy as np
    s = WL.spec(config)
    q, k, v = WL.make_rows(s)
    p = fs.params_to_device(WL.make_params(s))
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]

    def up(x):
        return torch.from_numpy(WL.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = up(q), up(k), up(v)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    go = torch.randn(qd.shape, generator=g, device="cuda").to(torch.bfloat16)
    dims = fs.make_dims(B, N, H, d, M, W, "bf16", "auto")
    nbytes = fs.idattn_backward_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = {"q": torch.empty_like(qd), "k": torch.empty_like(kd), "v": torch.empty_like(vd)}
    for key in fs.PARAM_KEYS:
        out[key] = torch.empty_like(p[key])
    gp = fs.make_param_grads(out)
    prm = fs.make_params(p)

    def call():
        fs.idattn_backward(dims, prm, qd, kd, vd, None, None, go, None, out["q"], out["k"], out["v"], gp, None, ws,
                           nbytes)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 7 * B * N * H * d * 2  # q, k, v and grad_o read once; grad_q, grad_k, grad_v written once (bf16)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{config}: B={B} H={H} N={N} d=R={d} M={M} W={W}, bf16 I/O, gradients of q, k, v and every "
                        f"parameter, sequential fp32 algorithm", "ms_per_call": ms, "tokens_per_s": B * N / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes": nbytes,
                         "note": "the sequential scans are serial in time; the algorithmic bytes are the tensors "
                                 "read and written once"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the mixer forward needs no "
              f"collective and this build runs on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fixed_state_ssm_amd as fs
    import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fs.load_library()
    if args.only:
        part = {"varlen": lambda: varlen_bench(torch, fs, WL),
                "normalized": lambda: normalized_bench(torch, fs, WL, args.config),
                "rff": lambda: rff_bench(torch, fs, WL, args.config),
                "backward": lambda: backward_bench(torch, fs, WL, args.config),
                "decode": lambda: decode_bench(torch, fs, steps=20, warmup=20)}[args.only]()
        print(json.dumps({args.only: part}), flush=True)
        return
    s = WL.spec(args.config)
    B, N, H, d, M, W = s["B"], s["N"], s["H"], s["d"], s["M"], s["W"]
    q, k, v = WL.make_rows(s)
    params = WL.make_params(s)
    if args.feature_norm == "rff":
        params["rff_omega"] = WL.make_rff_omega(s)
    p = fs.params_to_device(params)
    prm = fs.make_params(p)

    def up(x):
        return torch.from_numpy(WL.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    sets = []
    base = [up(q), up(k), up(v)]
    for r in range(3):
        sets.append([t.clone() for t in base] + [torch.empty_like(base[0])])
    del base
    state_out = torch.empty((B, H, M, 2 * d, 2), dtype=torch.float32, device="cuda")
    tail_out = torch.empty((B, H, 2, W - 1, d), dtype=torch.bfloat16, device="cuda")
    dims = fs.make_dims(B, N, H, d, M, W, "bf16", args.algo, feature_norm=args.feature_norm)
    nbytes = fs.idattn_forward_workspace_size(dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    algo = args.algo
    if algo == "auto":
        try:
            fs.idattn_forward_workspace_size(fs.make_dims(B, N, H, d, M, W, "bf16", "chunked",
                                                          feature_norm=args.feature_norm))
            algo = "chunked"
        except fs.IdattnError:
            algo = "sequential"

    def step(i):
        qq, kk, vv, oo = sets[i % len(sets)]
        fs.idattn_forward(dims, prm, qq, kk, vv, oo, None, None, state_out, tail_out, ws, nbytes)

    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            step(settle)
            settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for i in range(args.steps):
        step(i)
    r1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mean_launch_ms = r0.elapsed_time(r1) / args.steps
    wall = t1 - t0
    tokens = B * N * args.steps
    alg_bytes = B * N * H * d * 2 * 4
    achieved = alg_bytes / (mean_launch_ms * 1e-3) / 1e9
    flops_literal = 14.0 * M * 2 * d * B * N * H
    flops_mfma = chunked_mfma_flops(B, N, H, d) if algo == "chunked" else 0.0

    out = {
        "metric": METRIC,
        "value": tokens / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if algo == "sequential" else "f16-mfma/f32",
        "data": "synthetic (seeded N(0,1) bf16 q,k,v; S4D-Lin init)",
        "config": {"workload": f"{args.config}: B={B} H={H} N={N} d=R={d} M={M} W={W}, bf16 I/O, fp32 state"
                               + {"squared": "", "unit": ", unit-norm feature map",
                                  "rff": ", random Fourier feature map"}[args.feature_norm],
                   "B": B, "N": N, "H": H, "d": d, "M": M, "W": W, "io": "bf16", "algo": algo,
                   "feature_norm": args.feature_norm},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": committed_traffic(args.config, algo),
                     "kernel": "idattn_forward launch (all kernels of one forward; HIP events on the launch "
                               "stream around the timed launches, divided by their number)",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "launch_ms_mean": mean_launch_ms},
        "flops": {"literal_per_launch": flops_literal,
                  "literal_tflops": flops_literal / (mean_launch_ms * 1e-3) / 1e12,
                  "note": "the literal recurrence's flops are what the method defines, not what the chunked "
                          "kernels execute; mfma_* counts the matrix-core work the kernels issue",
                  "mfma_executed_per_launch": flops_mfma,
                  "mfma_tflops": flops_mfma / (mean_launch_ms * 1e-3) / 1e12,
                  "mfma_frac_fp16_peak": flops_mfma / (mean_launch_ms * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS},
        "settle_launches": settle,
        "source_sha": source_sha(),
    }
    out["measured_copy_gbps"] = measure_copy_gbps(torch)
    if not args.no_decode:
        out["decode"] = decode_bench(torch, fs, steps=20, warmup=20)
        out["decode"]["measured_inplace_stream_gbps"] = measure_inplace_gbps(torch)
        out["varlen"] = varlen_bench(torch, fs, WL, mean_launch_ms if args.config == "1p3b" else None)
        out["normalized"] = normalized_bench(torch, fs, WL, args.config, mean_launch_ms)
        out["rff"] = rff_bench(torch, fs, WL, args.config, mean_launch_ms)
        out["backward"] = backward_bench(torch, fs, WL, args.config)
    del sets, ws
    torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(s, q, k, v, params, args.cpu_seconds, args.feature_norm)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
