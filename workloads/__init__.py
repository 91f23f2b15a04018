"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only draws random inputs; it holds none of the layer's arithmetic
(no routing, no projection, no activation, no combine). It is shared by the
FP64 oracle's tests, the GPU parity tests and the benchmark, which is the one
thing the oracle and the HIP path are allowed to share.

Workload shapes follow the model shapes the pages name:
  * Qwen-3-style decode (warp-decode article, "Key points"): H=2048, E=128,
    k=8, I=768.  k*H*2 B = 32 KiB per token, the figure that article gives for
    the intermediate traffic warp decode removes.
  * Qwen3.5-397B-A17B (MoK summary, "What is 2.37x measured against"): 512
    experts, top-k 10.
  * Kimi K2.7 Code (same passage): 384 experts, hidden 7168.
  * DeepSeek-V4-Pro (same passage): 384 experts, intermediate 3072.
  * 2,048 tokens per GPU and expert-parallel degree 64 (same passage).
The remaining sizes (I for Kimi, H for DeepSeek, I for Qwen3.5) are assumed.

Recipe (every tensor from its own seeded stream, so one expert can be
regenerated alone):
  * activations x ~ N(0, sx^2) drawn in float32, rounded to BF16 (RNE);
  * weights ~ N(0, 0.02^2) drawn in float32, rounded to BF16 (RNE), or, for
    the MXFP8 workloads, stored as E4M3 codes with one E8M0 scale code per 32
    elements along K.  The weight scale exponent is the smallest s with
    448 * 2^s >= the block's max |w| (so no weight code saturates); the codes
    are torch's round-to-nearest-even float8_e4m3fn cast of w / 2^s.  This is
    how the synthetic parameters are made, not part of the layer;
  * router logits ~ N(0, 1) in float32; the Zipf workload adds a per-expert
    bias -1.1 * ln(rank_e), rank being a seeded permutation of 1..E.
Random draws use torch generators on the requested device; data made on the
GPU and data made on the CPU for the same seed differ, and each test uses one.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "get", "make", "make_weights", "make_activations",
           "expert_bytes"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    dtype: str = "bf16"        # "bf16" or "mxfp8"
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: float = 0.0        # 0 = no bias
    path: str = "decode"       # "decode" or "batched"
    note: str = ""

    def with_T(self, T: int) -> "Config":
        return dataclasses.replace(self, T=T, name=f"{self.name}@T{T}")


def _c(**kw) -> Config:
    return Config(**kw)


CONFIGS: Dict[str, Config] = {c.name: c for c in [
    _c(name="tiny-T4", T=4, H=512, E=8, k=2, I=256, x_std=0.02,
       note="tiny decode layer; oracle runs in well under a second"),
    _c(name="qwen3-decode-T1", T=1, H=2048, E=128, k=8, I=768,
       note="Qwen3-style decode, near-uniform routing"),
    _c(name="qwen3-decode-T8", T=8, H=2048, E=128, k=8, I=768,
       note="Qwen3-style decode, near-uniform routing"),
    _c(name="qwen3-decode-T32", T=32, H=2048, E=128, k=8, I=768,
       note="Qwen3-style decode, near-uniform routing"),
    _c(name="qwen3-mxfp8-decode-T32", T=32, H=2048, E=128, k=8, I=768, dtype="mxfp8",
       path="batched", note="Qwen3-style decode with MXFP8 weights (x and h MX-quantized), "
                            "served by the batched MXFP8 calls"),
    _c(name="q35-zipf-T64", T=64, H=4096, E=512, k=10, I=1024, zipf_s=1.1,
       note="Qwen3.5-397B-A17B-shaped decode, Zipf(1.1) expert skew"),
    _c(name="kimi-bf16-T2048", T=2048, H=7168, E=384, k=8, I=2048, path="batched",
       note="Kimi-K2.7-Code-shaped batched layer, all 384 experts resident"),
    _c(name="dsv4-mxfp8-T2048", T=2048, H=7168, E=384, k=8, I=3072, dtype="mxfp8",
       path="batched", note="DeepSeek-V4-Pro-shaped batched layer, MXFP8"),
    _c(name="glm-bf16-T2048", T=2048, H=6144, E=256, k=8, I=2048, path="batched",
       note="GLM-5.2-shaped batched layer (E and H from the pages; k = 8 and I = 2048 assumed)"),
    _c(name="kimi-bf16-ep64share", T=16384, H=7168, E=6, k=1, I=2048, path="batched",
       note="one GPU's share under expert parallelism 64 at 2048 tokens/GPU: "
            "16384 received rows over 384/64 = 6 local experts"),
    _c(name="dsv4-mxfp8-ep64share", T=16384, H=7168, E=6, k=1, I=3072, dtype="mxfp8",
       path="batched", note="MXFP8 one-GPU share under expert parallelism 64"),
]}

# stream tags: each tensor kind draws from its own stream
_TAG = {"x": 1, "logits": 2, "zipf": 3, "w_gate_up": 4, "w_down": 5, "dout": 6}


def get(name: str) -> Config:
    if name in CONFIGS:
        return CONFIGS[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")


def _seed(seed: int, tag: str, index: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), _TAG[tag], int(index)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device, seed: int, tag: str, index: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, index))
    return g


def _normal(shape, std, device, seed, tag, index=0) -> torch.Tensor:
    g = _gen(device, seed, tag, index)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _to_mxfp8(w: torch.Tensor):
    """Store float32 weights [..., K] as E4M3 codes + E8M0 scale codes (blocks
    of 32 along K), all leading rows at once.  Scale: smallest s with
    448 * 2^s >= block max |w|, decided exactly from the binary exponent of the
    max (no logarithms)."""
    K = w.shape[-1]
    lead = w.shape[:-1]
    blocks = w.reshape(-1, K // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    mant, expo = torch.frexp(amax)            # amax = mant * 2^expo, mant in [0.5, 1)
    # 448 * 2^(expo-9) = 0.875 * 2^expo  >= amax  <=>  mant <= 0.875
    s = torch.where(mant <= 0.875, expo - 9, expo - 8)
    s = torch.where(amax == 0, torch.full_like(s, -127), s).clamp(-127, 127)
    scaled = blocks * torch.pow(2.0, -s.to(torch.float32)).unsqueeze(-1)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, K)
    scales = (s + 127).to(torch.uint8).reshape(*lead, K // 32)
    return codes.contiguous(), scales.contiguous()


# float32 elements drawn before one vectorised MX quantization (1 GiB)
_MX_CHUNK_ELEMS = 1 << 28


def make_weights(cfg: Config, seed: int = 0, device="cpu", experts=None) -> Dict[str, torch.Tensor]:
    """Expert weights: w_gate_up [E, 2I, H] (gate rows [0, I), up rows [I, 2I)),
    w_down [E, H, I]; K (the reduction dim) contiguous.  BF16 tensors, or uint8
    E4M3 codes plus uint8 E8M0 scale codes [.., K/32] for MXFP8 workloads.
    ``experts`` restricts generation to a subset (others left zero).
    Each expert's values come from its own seeded stream; MXFP8 experts are
    drawn into a float32 chunk of several experts that is quantized in one
    pass, so the number of device operations does not grow with E."""
    E, H, I = cfg.E, cfg.H, cfg.I
    ids = list(range(E)) if experts is None else [int(e) for e in experts]
    out: Dict[str, torch.Tensor] = {}
    for name, (R, K) in (("w_gate_up", (2 * I, H)), ("w_down", (H, I))):
        if cfg.dtype == "bf16":
            buf = torch.zeros(E, R, K, dtype=torch.bfloat16, device=device)
            for e in ids:
                buf[e].copy_(_normal((R, K), cfg.w_std, device, seed, name, e).to(torch.bfloat16))
            out[name] = buf
        elif cfg.dtype == "mxfp8":
            codes = torch.zeros(E, R, K, dtype=torch.uint8, device=device)
            scales = torch.zeros(E, R, K // 32, dtype=torch.uint8, device=device)
            per = max(1, _MX_CHUNK_ELEMS // (R * K))
            stage = torch.empty(min(per, max(len(ids), 1)), R, K, dtype=torch.float32,
                                device=device)
            for c0 in range(0, len(ids), per):
                chunk = ids[c0:c0 + per]
                for i, e in enumerate(chunk):
                    torch.randn((R, K), generator=_gen(device, seed, name, e), out=stage[i])
                f = stage[:len(chunk)]
                if cfg.w_std != 1.0:
                    f.mul_(cfg.w_std)
                c, s = _to_mxfp8(f)
                sel = torch.as_tensor(chunk, device=device)
                codes.index_copy_(0, sel, c)
                scales.index_copy_(0, sel, s)
                del c, s
            out[name] = codes
            out[name + "_scales"] = scales
        else:
            raise ValueError(cfg.dtype)
    return out


def make_activations(cfg: Config, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """x [T, H] BF16 and router logits [T, E] float32."""
    x = _normal((cfg.T, cfg.H), cfg.x_std, device, seed, "x").to(torch.bfloat16)
    logits = _normal((cfg.T, cfg.E), 1.0, device, seed, "logits")
    if cfg.zipf_s:
        g = _gen("cpu", seed, "zipf")
        rank = torch.randperm(cfg.E, generator=g).to(torch.float64) + 1.0
        bias = (-cfg.zipf_s * torch.log(rank)).to(torch.float32).to(device)
        logits = logits + bias
    return {"x": x.contiguous(), "logits": logits.contiguous()}


def make_output_grad(cfg: Config, seed: int = 0, device="cpu") -> torch.Tensor:
    """Gradient of the layer output for the backward pass: dout [T, H] BF16,
    N(0, 1) (the scale of a loss gradient does not change relative errors)."""
    return _normal((cfg.T, cfg.H), 1.0, device, seed, "dout").to(torch.bfloat16).contiguous()


def make(name_or_cfg, seed: int = 0, device="cpu", T: Optional[int] = None) -> Dict[str, object]:
    cfg = get(name_or_cfg) if isinstance(name_or_cfg, str) else name_or_cfg
    if T is not None and T != cfg.T:
        cfg = cfg.with_T(T)
    d: Dict[str, object] = {"cfg": cfg}
    d.update(make_activations(cfg, seed, device))
    d.update(make_weights(cfg, seed, device))
    return d


def expert_bytes(cfg: Config) -> int:
    """Bytes of one expert's weights (gate, up and down), including MXFP8
    scale codes."""
    n = 3 * cfg.H * cfg.I
    if cfg.dtype == "bf16":
        return 2 * n
    return n + n // 32


def _self_check():  # pragma: no cover - manual
    for c in CONFIGS.values():
        print(c.name, c.T, c.H, c.E, c.k, c.I, c.dtype, f"{c.E * expert_bytes(c) / 1e9:.2f} GB")


if __name__ == "__main__":  # pragma: no cover
    _self_check()
