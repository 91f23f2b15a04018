"""CPU checks of the GPU tests' helpers (tests/_gpu.py): the threaded,
pre-decoded way they run the oracle gives exactly the oracle's own result, and
the token sampler covers what it promises."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_backward, moe_forward, route
from tests import _gpu as G


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _cfg(dtype, T=24, H=256, I=256, E=6, k=2):
    return W.Config(name=f"helper-{dtype}", T=T, H=H, E=E, k=k, I=I, dtype=dtype, path="batched")


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
@pytest.mark.parametrize("tokens", [None, [0, 3, 7, 20]])
def test_oracle_helper_equals_plain_oracle(dtype, tokens):
    d = W.make(_cfg(dtype), seed=5, device="cpu")
    cfg = d["cfg"]
    kw = {}
    if dtype == "mxfp8":
        kw = dict(w_gate_up_scales=d["w_gate_up_scales"].numpy(),
                  w_down_scales=d["w_down_scales"].numpy())
        wgu, wd = d["w_gate_up"].numpy(), d["w_down"].numpy()
    else:
        wgu, wd = _bits(d["w_gate_up"]), _bits(d["w_down"])
    want, wi = moe_forward(_bits(d["x"]), d["logits"].numpy(), wgu, wd, cfg.k, dtype=dtype,
                           tokens=tokens, return_intermediates=True, **kw)
    got, gi = G.oracle(d, tokens=tokens, return_intermediates=True)
    assert np.array_equal(got, want)                  # bit-identical float64
    assert np.array_equal(gi["a"], wi["a"]) and np.array_equal(gi["idx"], wi["idx"])


def test_backward_helper_equals_plain_oracle():
    d = W.make(_cfg("bf16", T=40, E=5, k=2), seed=8, device="cpu")
    cfg = d["cfg"]
    dout = W.make_output_grad(cfg, seed=2)
    for tokens, experts in ((None, None), ([1, 5, 30], [0, 3])):
        want = moe_backward(_bits(d["x"]), d["logits"].numpy(), _bits(d["w_gate_up"]),
                            _bits(d["w_down"]), _bits(dout), cfg.k, tokens=tokens,
                            experts=experts)
        got = G.oracle_backward(d, dout, tokens=tokens, experts=experts)
        for key in ("dx", "d_topk_w", "dlogits", "dw_gate_up", "dw_down"):
            assert np.array_equal(got[key], want[key]), key


def test_decoded_serves_out_of_order_requests():
    w = torch.randn(5, 8, 32).to(torch.bfloat16)
    dec = G.Decoded(w, None, order=[0, 2, 4], window=2)
    for e in (4, 1, 0, 2, 3):                       # including ids outside `order`
        assert np.array_equal(dec(e), G.F.bf16_decode(_bits(w[e])))


def test_sample_tokens_covers_extremes_and_ragged_tiles():
    g = torch.Generator().manual_seed(3)
    logits = torch.randn(2048, 96, generator=g)
    logits[:, 5] += 1.5                              # a heavy expert
    lg = logits.numpy()
    k = 4
    toks, info = G.sample_tokens(lg, k, 64, seed=1)
    assert toks.size >= 64 and np.all(np.diff(toks) > 0) and toks.max() < 2048
    idx, _ = route(lg, k)
    counts = np.bincount(idx.ravel(), minlength=96)
    assert info["heavy"] == int(np.argmax(counts))
    used = np.nonzero(counts)[0]
    assert counts[info["light"]] == counts[used].min()
    for e in (info["heavy"], info["light"]):
        mine = np.nonzero((idx == e).any(axis=1))[0]
        assert mine[0] in toks and mine[-1] in toks
        for bm in (64, 128, 256):
            assert mine[(mine.size - 1) // bm * bm] in toks    # first row of the last M-tile
    # deterministic for a seed
    assert np.array_equal(G.sample_tokens(lg, k, 64, seed=1)[0], toks)
