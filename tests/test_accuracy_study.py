"""Accuracy study of the hand-off between the two projections (the analogue of
the warp-decode article's "Comparison": keeping the intermediate activations
unquantized brought its output closer to an FP32 reference).

For the Qwen3-style decode shape, the FP64 oracle computes the layer three
ways - exact, with the gated activations rounded to BF16 before the down
projection (this library's decode hand-off), and with them MX-quantized to FP8
(E4M3 + E8M0 per 32, an FP8 intermediate) - each output rounded once to BF16
as the library's output is.  The test pins the ordering and the size of the gap;
the GPU decode path's own distance is measured beside it in
tests/test_gpu_decode.py::test_decode_accuracy_study."""
import numpy as np
import torch

import workloads as W
from oracle import moe_forward, route
from oracle.moe import rel_l2
from oracle.formats import bf16_round


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def study(name: str = "qwen3-decode-T8", tokens: int = 2, seed: int = 0):
    cfg = W.get(name)
    act = W.make_activations(cfg, seed)
    logits = act["logits"][:tokens].numpy()
    touched = sorted(set(route(logits, cfg.k)[0].ravel().tolist()))
    wts = W.make_weights(cfg, seed, experts=touched)
    x = _bits(act["x"][:tokens])
    wgu, wd = _bits(wts["w_gate_up"]), _bits(wts["w_down"])
    exact = moe_forward(x, logits, wgu, wd, cfg.k)
    dist = {}
    for mode in ("exact", "bf16", "mxfp8"):
        out = exact if mode == "exact" else moe_forward(x, logits, wgu, wd, cfg.k, h_round=mode)
        dist[mode] = rel_l2(bf16_round(out), exact)
    return dist


def test_bf16_hand_off_is_closer_than_fp8():
    d = study()
    print(f"[accuracy] rel-L2 to FP64, BF16 output: exact h {d['exact']:.3e}, "
          f"BF16 h {d['bf16']:.3e}, MXFP8 h {d['mxfp8']:.3e} "
          f"(FP8 / BF16 = {d['mxfp8'] / d['bf16']:.2f})")
    # the output rounding alone costs ~2^-9 relative; a BF16 hand-off adds a
    # little on top, an FP8 one (3 mantissa bits) several times more
    assert d["exact"] < d["bf16"] < d["mxfp8"]
    assert d["bf16"] < 1.5 * d["exact"]
    assert d["mxfp8"] > 3 * d["bf16"]
