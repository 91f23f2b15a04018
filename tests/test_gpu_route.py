"""GPU parity of moe_route_topk against the oracle's routing: indices bit-exact,
weights within 1e-6."""
import numpy as np
import pytest
import torch

from oracle import route
from tests._gpu import W_ABS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def _check(M, logits: torch.Tensor, k: int, what: str):
    print(f"[route] {what} T={logits.shape[0]} E={logits.shape[1]} k={k}", flush=True)
    idx, w = M.moe_route_topk(logits.cuda().contiguous(), k)
    torch.cuda.synchronize()
    ridx, rw = route(logits.cpu().numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ridx), what
    assert np.max(np.abs(w.cpu().double().numpy() - rw)) <= W_ABS, what


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 8, 2), (33, 128, 8), (64, 512, 10),
                                   (2048, 384, 8), (1000, 1024, 32), (300, 64, 64 // 2),
                                   (17, 6, 6), (5, 3, 1), (16384, 6, 1)])
def test_route_random(M, T, E, k):
    g = torch.Generator().manual_seed(T * 7 + E)
    _check(M, torch.randn(T, E, generator=g), k, "normal")


def test_route_ties_and_signed_zero(M):
    g = torch.Generator().manual_seed(1)
    grid = (torch.randint(-3, 4, (500, 40), generator=g) / 2.0).float()   # many exact ties
    _check(M, grid, 7, "grid")
    z = torch.zeros(8, 16)
    z[::2, 3] = -0.0
    z[1::2, 5] = -0.0
    _check(M, z, 4, "zeros")
    l = torch.tensor([[-0.0, 0.0, -1.0, 0.0]]).repeat(3, 1)
    _check(M, l, 2, "signed zero")
    big = torch.full((4, 70), -3.4e38)
    big[:, 69] = 3.4e38
    _check(M, big, 3, "extremes")


def test_route_empty_batch(M):
    idx, w = M.moe_route_topk(torch.empty(0, 8, device="cuda"), 2)
    assert idx.shape == (0, 2)


def test_route_deterministic(M):
    l = torch.randn(2048, 384, device="cuda")
    a = M.moe_route_topk(l, 8)
    for _ in range(3):
        b = M.moe_route_topk(l, 8)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
