"""Helpers shared by the GPU parity tests: move data to the oracle, run it, compare."""
import numpy as np
import torch

from oracle import moe_forward
from oracle.moe import max_abs_ratio, rel_l2

BF16_REL_L2 = 5e-3          # relative L2 bound for BF16 outputs
BF16_MAX_ABS = 1e-2         # max |got - ref| <= this * max |ref|
MXFP8_REL_L2 = 3e-2         # relative L2 bound for MXFP8 outputs (quantization-aware oracle)
W_ABS = 1e-6                # routing weights: FP32 path vs FP64 oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


class Fetch:
    """Callable e -> one expert's weights as numpy, copied from the GPU on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __call__(self, e):
        w = self.t[int(e)]
        return bits(w) if w.dtype == torch.bfloat16 else u8(w)


def oracle(d, tokens=None, return_intermediates=False):
    """Run the FP64 oracle on a workload dict (tensors may live on the GPU)."""
    cfg = d["cfg"]
    kw = {}
    if cfg.dtype == "mxfp8":
        kw = dict(w_gate_up_scales=Fetch(d["w_gate_up_scales"]),
                  w_down_scales=Fetch(d["w_down_scales"]))
    return moe_forward(bits(d["x"]), d["logits"].detach().cpu().numpy(), Fetch(d["w_gate_up"]),
                       Fetch(d["w_down"]), cfg.k, dtype=cfg.dtype, tokens=tokens,
                       return_intermediates=return_intermediates, **kw)


def to_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().cpu().double().numpy()


def check_bf16(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = to_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rl, ma = rel_l2(g, ref), max_abs_ratio(g, ref)
    print(f"[parity] {what}: rel_l2={rl:.3e} max_abs/max={ma:.3e}", flush=True)
    assert rl <= BF16_REL_L2, f"{what}: rel_l2 {rl:.3e} > {BF16_REL_L2}"
    assert ma <= BF16_MAX_ABS, f"{what}: max-abs ratio {ma:.3e} > {BF16_MAX_ABS}"
    return rl, ma
