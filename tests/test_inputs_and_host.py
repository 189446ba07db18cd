"""CPU checks of the seeded input generator and of the host-side work model."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from rankmixer_token_mixing_amd import perfmodel as pm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_generator_is_deterministic_and_shaped():
    cfg = si.scaled(si.CONFIGS["c1"], B=8, T=4, D=64, L=2)
    a = si.make_inputs(cfg)
    b = si.make_inputs(cfg)
    assert a["x"].dtype == np.uint16 and a["x"].shape == (8, 4, 64)
    np.testing.assert_array_equal(a["x"], b["x"])
    for blk_a, blk_b in zip(a["blocks"], b["blocks"]):
        for k in blk_a:
            np.testing.assert_array_equal(blk_a[k], blk_b[k])
    assert a["blocks"][0]["w1"].shape == (4, 256, 64)
    assert a["blocks"][0]["w2"].shape == (4, 64, 256)
    assert not np.array_equal(a["blocks"][0]["w1"], a["blocks"][1]["w1"])
    c = si.make_inputs(cfg, seed=7)
    assert not np.array_equal(a["x"], c["x"])


def test_generator_statistics():
    cfg = si.scaled(si.CONFIGS["c1"], B=64, T=4, D=256, L=1)
    a = si.make_inputs(cfg)
    x = si.bf16_bits_to_f32(a["x"]).astype(np.float64)
    assert abs(x.std() - 1.0) < 0.01
    w1 = si.bf16_bits_to_f32(a["blocks"][0]["w1"]).astype(np.float64)
    assert abs(w1.std() * math.sqrt(256) - 1.0) < 0.01
    w2 = si.bf16_bits_to_f32(a["blocks"][0]["w2"]).astype(np.float64)
    assert abs(w2.std() * math.sqrt(1024) - 1.0) < 0.01
    assert abs(a["blocks"][0]["b1"].std() - 0.1) < 0.01   # N(0, 0.01) is variance 0.01


def test_generator_bf16_rounding_is_torch_rne():
    x = (np.random.default_rng(0).standard_normal(100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(si.to_bf16_bits(x), ref)


def test_generator_chunks_are_thread_count_independent(monkeypatch):
    monkeypatch.setattr(si, "CHUNK", 1000)
    a = np.empty(5500, np.float32)
    si._fill_normal(a, 3, 0, 1.0)
    monkeypatch.setattr(si, "_threads", lambda: 1)
    b = np.empty(5500, np.float32)
    si._fill_normal(b, 3, 0, 1.0)
    np.testing.assert_array_equal(a, b)


def test_config_table_matches_the_workloads():
    c = si.CONFIGS
    assert (c["c0"].B, c["c0"].T, c["c0"].D, c["c0"].hidden, c["c0"].L, c["c0"].dtype) == (64, 4, 64, 128, 1, "f32")
    assert (c["c1"].B, c["c1"].T, c["c1"].D, c["c1"].hidden, c["c1"].L) == (2048, 16, 768, 3072, 2)
    assert (c["c2"].B, c["c2"].T, c["c2"].D, c["c2"].F, c["c2"].L, c["c2"].head) == (4096, 16, 320, 5000, 4, True)
    assert (c["c3"].B, c["c3"].T, c["c3"].D, c["c3"].hidden, c["c3"].L) == (1024, 32, 1536, 6144, 2)
    assert (c["c4"].B, c["c4"].T, c["c4"].D, c["c4"].E, c["c4"].He, c["c4"].L) == (2048, 16, 768, 8, 1536, 2)
    for cfg in c.values():
        assert cfg.D % cfg.T == 0


def test_flop_convention_reproduces_appendix_b():
    g = json.load(open(os.path.join(GOLDEN, "appendix_b_flops.json")))
    B, n, L = g["batch"], g["width"], g["layers"]
    got = {
        "dcn": pm.dcn_flops(B, n, L),
        "dcnv2_rank32": pm.dcnv2_lowrank_flops(B, n, g["dcnv2_rank"], L),
        "dcnv2_full": pm.dcnv2_full_flops(B, n, L),
        "mixer_bmm": pm.mixer_backbone_flops(B, g["mixer_tokens"], g["mixer_token_width"], g["mixer_hidden"], L),
    }
    for k, v in got.items():
        assert round(v / 1e9, 6) == pytest.approx(g["gflops"][k], abs=1.5e-6), k
    # the printed throughputs are the printed flops over the printed times
    for k in ("mixer_bmm", "mixer_loop", "dcnv2_full"):
        assert g["gflops"][k] / g["timing_ms"][k] == pytest.approx(g["tflops"][k], rel=2e-3)


def test_block_param_and_flop_counts():
    # 2*T*k*D^2 weights per block; ~1.2B for the two 1B-class blocks
    assert pm.block_params(32, 1536, 4) * 2 == 1_207_959_552
    assert pm.block_flops(1, 32, 1536, 6144) == 1_207_959_552
    assert pm.block_flops(1024, 32, 1536, 6144) == 1_236_950_581_248
    # MoE at every expert active equals a dense block of width E*He plus the router
    assert pm.moe_flops(16 * 8, 1, 16, 768, 8, 1536) == pm.block_flops(1, 16, 768, 8 * 1536) + 16 * 2 * 8 * 768
