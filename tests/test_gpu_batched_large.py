"""GPU parity of the large-group batched GEMMs (taken when the routed rows per
expert average at least 256: the MFMA-bound regime of one GPU's
expert-parallel share) against the FP64 oracle, BF16.

The shapes are small enough for the oracle to check every token, and large
enough that P = T*k >= 256*E, so the 256-row tiles run: several M-tiles per
expert with a ragged last tile, several N-blocks, K loops of 4..12 stages,
both down epilogues (k = 1 writes the output directly, k > 1 goes through the
FP32 slots and the fixed-order combine)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import route
from tests._gpu import check_bf16, oracle
from tests.test_gpu_batched import _check, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def _custom(T, H, I, E, k, seed=0):
    cfg = W.Config(name=f"bl-T{T}-H{H}-I{I}-E{E}-k{k}", T=T, H=H, E=E, k=k, I=I, x_std=1.0,
                   path="batched")
    return W.make(cfg, seed=seed, device="cuda")


@pytest.mark.parametrize("T,H,I,E,k", [
    (600, 256, 256, 2, 1),      # 2 M-tiles per expert (ragged), k = 1
    (1100, 256, 256, 4, 1),     # 4 experts, ~275 rows each
    (520, 768, 256, 2, 1),      # 12 K stages in gate_up, 3 N-blocks in down
    (300, 512, 512, 2, 2),      # k = 2: FP32 slots + combine, 4 N-blocks in gate_up
    (300, 256, 256, 2, 2),      # k = E
])
def test_large_shapes(M, T, H, I, E, k):
    assert T * k >= 256 * E
    _check(M, _custom(T, H, I, E, k, seed=T + 7 * E), f"large shape T={T} H={H} I={I} E={E} k={k}")


def test_large_all_on_one_expert(M):
    # every token on expert 0 (3 M-tiles), expert 1 empty
    d = _custom(700, 256, 256, 2, 1, seed=11)
    lg = d["logits"]
    lg[:, 0] = 5.0
    lg[:, 1] = -5.0
    _check(M, d, "large: all tokens on one expert")


def test_large_bit_identical_repeats(M):
    d = _custom(1100, 256, 256, 4, 2, seed=5)
    first = run_layer(M, d)
    for _ in range(4):
        again = run_layer(M, d)
        assert torch.equal(again[0].view(torch.int16), first[0].view(torch.int16))
        assert torch.equal(again[3].view(torch.int16), first[3].view(torch.int16))


def test_large_h_rows_grouped(M):
    # h comes out in sorted-row order (expert ascending, token ascending)
    d = _custom(600, 256, 256, 2, 1, seed=4)
    cfg = d["cfg"]
    out, idx, w, h, ws = run_layer(M, d)
    ridx, _ = route(d["logits"].cpu().numpy(), cfg.k)
    pairs = sorted((int(ridx[t, j]), t, j) for t in range(cfg.T) for j in range(cfg.k))
    _, inter = oracle(d, return_intermediates=True)
    want = np.stack([inter["a"][t, j] for (_, t, j) in pairs])
    got = h.float().cpu().double().numpy()
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 5e-3, rel


def test_large_whole_rounds_without_split(M):
    # tokens dealt round-robin to 4 experts: 1,024 rows each = 4 tiles, so gate_up has
    # exactly 16 tiles x 16 N-blocks = 256 items (no tail to split), down 16 items (split)
    T, E = 4096, 4
    d = _custom(T, 256, 2048, E, 1, seed=21)
    lg = torch.full((T, E), -4.0, device="cuda")
    lg[torch.arange(T), torch.arange(T) % E] = 4.0
    d["logits"] = lg.contiguous()
    tokens = np.sort(np.random.default_rng(2).choice(T, size=192, replace=False))
    _check(M, d, "large: whole rounds (no tail split)", tokens=tokens)
