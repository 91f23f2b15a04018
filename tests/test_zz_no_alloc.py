"""The entry point that allocates nothing (moe_decode_forward_noalloc) against
the one it is a variant of (moe_decode_forward, caller workspace): the same
bytes, on two calls in a row, the second with a smaller batch (the shared
scratch array keeps the first call's contents), and both within the parity
bars of the FP64 oracle.  Its size limit is checked on the host."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import route
from tests._gpu import check_bf16, oracle


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def _run_both(M, d):
    cfg = d["cfg"]
    T, H, k = cfg.T, cfg.H, cfg.k
    outs = []
    for fn in ("moe_decode_forward", "moe_decode_forward_noalloc"):
        out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        getattr(M, fn)(d["x"], d["logits"], d["w_gate_up"], d["w_down"], k, out=out,
                       topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        outs.append((out, idx, w))
    return outs


@pytest.mark.gpu
def test_noalloc_matches_decode_forward_on_two_calls(M):
    # first a 32-token batch, then a 4-token one into the same scratch array
    for name, T, seed in (("qwen3-decode-T32", 32, 11), ("qwen3-decode-T32", 4, 12),
                          ("q35-zipf-T64", 64, 13), ("tiny-T4", 1, 14)):
        print(f"[noalloc] {name} T={T} seed={seed}", flush=True)
        d = W.make(name, seed=seed, device="cuda", T=T)
        (o0, i0, w0), (o1, i1, w1) = _run_both(M, d)
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
        cfg = d["cfg"]
        assert np.array_equal(i1.cpu().numpy(), route(d["logits"].cpu().numpy(), cfg.k)[0])
        check_bf16(o1, oracle(d), f"noalloc {name} T={T}")


@pytest.mark.gpu
def test_noalloc_without_topk_outputs(M):
    d = W.make("qwen3-decode-T8", seed=21, device="cuda")
    cfg = d["cfg"]
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    M.moe_decode_forward_noalloc(d["x"], d["logits"], d["w_gate_up"], d["w_down"], cfg.k, out)
    ref = M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_limits_checked_on_the_host(M):
    # rejected before any HIP call: works without a GPU
    lib, FAKE = M.lib, 0x10000
    call = lambda T, H, I, E, k: lib.moe_decode_forward_noalloc(
        FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, FAKE, None, None, None)
    assert M.moe_decode_workspace_bytes(64, 2048, 2048, 128, 32) > M.STATIC_SCRATCH_BYTES
    assert call(64, 2048, 2048, 128, 32) == M.MOE_ERR_UNSUPPORTED
    assert b"scratch" in lib.moe_last_error()
    assert call(65, 2048, 768, 128, 8) == M.MOE_ERR_UNSUPPORTED
    assert call(4, 384, 256, 8, 2) == M.MOE_ERR_SHAPE
    assert lib.moe_decode_forward_noalloc(None, FAKE, FAKE, FAKE, 4, 512, 256, 8, 2, FAKE, None,
                                          None, None) == M.MOE_ERR_NULL
    assert lib.moe_decode_forward_noalloc(FAKE + 2, FAKE, FAKE, FAKE, 4, 512, 256, 8, 2, FAKE,
                                          None, None, None) == M.MOE_ERR_ALIGN
    # the largest page shape fits: Qwen3.5-shaped decode at T = 64 (k 10, I 1024)
    assert M.moe_decode_workspace_bytes(64, 4096, 1024, 512, 10) <= M.STATIC_SCRATCH_BYTES
