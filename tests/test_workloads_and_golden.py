"""Seeded input generator and the oracle's regression fixture (CPU only)."""
import json
import os

import numpy as np
import torch

import oracle
import workloads as WL

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_rounding_matches_torch_rne():
    r = np.random.default_rng(0)
    x = np.concatenate([r.normal(size=100000).astype(np.float32) * 10.0 ** r.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.3895e38, 1e-40], np.float32)]).astype(np.float32)
    ours = WL.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(WL.bf16_from_bits(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rows_regenerate_independently():
    s = WL.spec("125m", N=64)
    q, k, v = WL.make_rows(s)
    q2, k2, v2 = WL.make_rows(s, rows=[5, 2])
    assert np.array_equal(q[[5, 2]], q2) and np.array_equal(v[[5, 2]], v2)
    assert q.shape == (8, 64, 12, 64)
    assert np.array_equal(WL.bf16_round(q), q)  # stored values are bf16-exact


def test_param_distributions():
    s = WL.spec("1p3b")
    p = WL.make_params(s)
    assert p["conv_q"].shape == (16, 128, 4) and p["gain"].shape == (16, 256)
    assert abs(p["conv_q"].std() - 0.5) < 0.02 and abs(p["bias"].std() - 0.02) < 0.002
    dt = np.exp(p["log_dt"])
    assert dt.min() >= 1e-3 and dt.max() <= 1e-1
    assert np.all(p["A"][..., 0] == -0.5)
    assert np.allclose(p["A"][:, :, 1], np.pi * np.arange(64)[None], rtol=1e-6)
    assert np.all(p["Bc"][..., 0] == 1.0) and np.all(p["Bc"][..., 1] == 0.0)


def test_decode_draws():
    s = WL.spec("decode")
    qt, kt, vt = WL.make_decode_token(s, rows=[0, 255])
    assert qt.shape == (2, 16, 128)
    st, tl = WL.make_decode_state(s, rows=[3])
    assert st.shape == (1, 16, 64, 256) and tl.shape == (1, 16, 2, 3, 128)


def test_oracle_reproduces_golden():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        g = json.load(f)
    c = WL.make_case("tiny")
    o, st, _ = oracle.forward(c.q, c.k, c.v, c.params, g["eps_feat"], g["eps_norm"])
    for i in g["positions"]:
        np.testing.assert_allclose(o[0, i], np.array(g["o"][str(i)]), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(st[0, 0, 0].real, g["state_out_mode0_head0_re"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(st[0, 1, 5].imag, g["state_out_mode5_head1_im"], rtol=1e-12, atol=1e-15)
