"""Workload generator checks: determinism, shapes, dtypes, the Zipf bias, the
MXFP8 weight encoding, and the model shapes the pages print."""
import json
import os

import numpy as np
import torch

import workloads as W
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def test_shapes_follow_the_pages():
    g = json.load(open(GOLDEN))
    q = W.get("qwen3-decode-T8")
    assert q.k * q.H * 2 >= g["qwen3_intermediate_bytes_per_token_min"]["value"]
    assert q.k * q.H * 2 == 32768
    kimi = W.get("kimi-bf16-T2048")
    assert (kimi.E, kimi.H) == (g["kimi_k27_code"]["E"], g["kimi_k27_code"]["H"])
    q35 = W.get("q35-zipf-T64")
    assert (q35.E, q35.k) == (g["qwen35_397b_a17b"]["E"], g["qwen35_397b_a17b"]["k"])
    ds = W.get("dsv4-mxfp8-T2048")
    assert (ds.E, ds.I) == (g["deepseek_v4_pro"]["E"], g["deepseek_v4_pro"]["I"])
    glm = W.get("glm-bf16-T2048")
    assert (glm.E, glm.H) == (g["glm_52"]["E"], g["glm_52"]["H"])
    for c in (kimi, ds, glm):
        assert c.T == g["tokens_per_gpu"]["value"]
    # one GPU's share under EP 64: all 2048*k received rows over E/64 local experts
    for share, full in (("kimi-bf16-ep64share", kimi), ("dsv4-mxfp8-ep64share", ds)):
        s = W.get(share)
        assert s.E == full.E // g["ep_degree"]["value"]
        assert s.T == full.T * full.k and s.k == 1 and (s.H, s.I) == (full.H, full.I)


def test_deterministic_and_shapes():
    a = W.make("tiny-T4", seed=3)
    b = W.make("tiny-T4", seed=3)
    c = W.make("tiny-T4", seed=4)
    for key in ("x", "logits", "w_gate_up", "w_down"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    cfg = a["cfg"]
    assert a["x"].shape == (cfg.T, cfg.H) and a["x"].dtype == torch.bfloat16
    assert a["logits"].shape == (cfg.T, cfg.E) and a["logits"].dtype == torch.float32
    assert a["w_gate_up"].shape == (cfg.E, 2 * cfg.I, cfg.H)
    assert a["w_down"].shape == (cfg.E, cfg.H, cfg.I)
    x = a["x"].float()
    assert 0.01 < x.std().item() < 0.03          # N(0, 0.02^2) for the tiny layer


def test_single_expert_regenerates_alone():
    cfg = W.get("tiny-T4")
    full = W.make_weights(cfg, seed=5)
    one = W.make_weights(cfg, seed=5, experts=[6])
    assert torch.equal(full["w_gate_up"][6], one["w_gate_up"][6])
    assert torch.equal(full["w_down"][6], one["w_down"][6])
    assert one["w_gate_up"][5].abs().sum() == 0


def test_zipf_bias_form():
    cfg = W.get("q35-zipf-T64")
    small = W.Config(name="z", T=4000, H=64, E=cfg.E, k=cfg.k, I=32, zipf_s=1.1)
    plain = W.Config(name="z", T=4000, H=64, E=cfg.E, k=cfg.k, I=32)
    a = W.make_activations(small, seed=1)["logits"].double()
    b = W.make_activations(plain, seed=1)["logits"].double()
    bias = (a - b).mean(0).numpy()
    ranks = np.exp(-bias / 1.1)                    # recovers the seeded ranks 1..E
    assert np.allclose(np.sort(ranks), np.arange(1, cfg.E + 1), rtol=1e-4)


def test_mxfp8_weights_decode_close_and_never_saturate():
    cfg = W.Config(name="m", T=2, H=128, E=3, k=1, I=64, dtype="mxfp8")
    w = W.make_weights(cfg, seed=2)
    codes, scales = w["w_gate_up"].numpy(), w["w_gate_up_scales"].numpy()
    assert codes.shape == (3, 128, 128) and scales.shape == (3, 128, 4)
    assert not np.any((codes & 0x7F) == 0x7F)       # no NaN codes
    deq = F.mx_dequantize(codes, scales)
    src = torch.randn(128, 128, generator=W._gen("cpu", 2, "w_gate_up", 1)).double().numpy() * 0.02
    assert np.max(np.abs(deq[1] - src)) <= 0.07 * np.max(np.abs(src))
    # each block's max uses the top binade without passing 448
    top = np.abs(F.e4m3_decode(codes)).reshape(3, 128, 4, 32).max(-1)
    assert np.all((top >= 224) & (top <= 448))
