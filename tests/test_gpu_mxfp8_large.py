"""GPU parity of the MXFP8 large-group GEMMs (256-row tiles, taken when the
routed rows per expert average at least 256) against the quantization-aware
FP64 oracle: relative L2 within 3e-2 (tripwire 1e-2).

Shapes keep P = T*k >= 256*E.  With stages of 128 along K, H and I of 512 or
more let the last partial round split along K; H = 256 runs it whole."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import route
from oracle.moe import rel_l2
from tests._gpu import oracle
from tests.test_gpu_mxfp8 import _check, run_mx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def _custom(T, H, I, E, k, seed=0):
    cfg = W.Config(name=f"mxl-T{T}-H{H}-I{I}-E{E}-k{k}", T=T, H=H, E=E, k=k, I=I,
                   dtype="mxfp8", path="batched")
    return W.make(cfg, seed=seed, device="cuda")


@pytest.mark.parametrize("T,H,I,E,k", [
    (600, 256, 256, 2, 1),      # 2 M-tiles per expert (ragged); 2 stages, no split
    (600, 1024, 512, 2, 1),     # 8 stages in gate_up: the tail splits along K
    (1100, 512, 256, 4, 1),     # 4 experts
    (520, 768, 256, 2, 1),      # 6 stages in gate_up, 3 N-blocks in down
    (300, 512, 512, 2, 2),      # k = 2: FP32 slots + combine
])
def test_mx_large_shapes(M, T, H, I, E, k):
    assert T * k >= 256 * E
    _check(M, _custom(T, H, I, E, k, seed=T + 3 * E), f"mx large shape T={T} H={H} I={I} E={E} k={k}")


def test_mx_large_all_on_one_expert(M):
    d = _custom(700, 512, 256, 2, 1, seed=12)
    d["logits"][:, 0] = 5.0
    d["logits"][:, 1] = -5.0
    _check(M, d, "mx large: all tokens on one expert")


def test_mx_large_whole_rounds(M):
    # round-robin routing: 4 x 1,024 rows = 16 tiles x 16 N-blocks = 256 gate_up items
    T, E = 4096, 4
    d = _custom(T, 256, 2048, E, 1, seed=22)
    lg = torch.full((T, E), -4.0, device="cuda")
    lg[torch.arange(T), torch.arange(T) % E] = 4.0
    d["logits"] = lg.contiguous()
    tokens = np.sort(np.random.default_rng(3).choice(T, size=192, replace=False))
    _check(M, d, "mx large: whole rounds", tokens=tokens)


def test_mx_large_bit_identical_repeats(M):
    d = _custom(1100, 512, 256, 4, 2, seed=8)
    first = run_mx(M, d)
    for _ in range(3):
        again = run_mx(M, d)
        assert torch.equal(again[0].view(torch.int16), first[0].view(torch.int16))
        assert torch.equal(again[3], first[3]) and torch.equal(again[4], first[4])


def test_mx_large_h_codes(M):
    # h codes and scales from the large gate_up (whole and split tiles) are an MX
    # quantization of activations close to the oracle's
    d = _custom(600, 1024, 512, 2, 1, seed=13)
    cfg = d["cfg"]
    out, idx, w, h, hs = run_mx(M, d)
    codes, scales = h.cpu().numpy(), hs.cpu().numpy()
    deq = F.mx_dequantize(codes, scales)
    c2, s2 = F.mx_quantize(deq)
    assert np.array_equal(s2, scales) and np.array_equal(c2, codes)
    _, inter = oracle(d, return_intermediates=True)
    ridx, _ = route(d["logits"].cpu().numpy(), cfg.k)
    pairs = sorted((int(ridx[t, j]), t, j) for t in range(cfg.T) for j in range(cfg.k))
    want = np.stack([inter["a"][t, j] for (_, t, j) in pairs])
    assert rel_l2(deq, want) < 1e-2
