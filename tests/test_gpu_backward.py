"""GPU parity of the backward pass (moe_route_topk -> moe_backward_batched)
against the FP64 oracle (oracle/backward.py), BF16.

dx, dw_gate_up and dw_down are BF16 results of FP32 sums whose operands were
rounded to BF16 once (the recomputed SwiGLU activation, the scaled output
gradient, the gradient of [g; u]): the forward's bounds apply (relative L2
<= 5e-3, max-abs <= 1e-2 of the largest value).  d_topk_w and dlogits stay
in FP32 from FP32 operands; their bounds (1e-4 and 1e-3 relative L2, the
latter allowing for the cancellation in dw_m - sum_j w_j dw_j) are far above
FP32 rounding over sums of a few thousand terms.
Small shapes are checked in full; the full-size workloads on seeded samples
of tokens (dx, d_topk_w, dlogits: each row depends on its token alone) and of
experts (weight gradients: each depends on the rows routed to that expert)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.moe import rel_l2
from tests._gpu import check_bf16, oracle_backward, sample_tokens, to_f64

pytestmark = pytest.mark.gpu

DTW_REL_L2 = 1e-4
DLOGITS_REL_L2 = 1e-3


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def run_bwd(M, d, dout, saved=False):
    """Routing, then the backward pass; with saved=True the gate/up pre-activations
    come from moe_gate_up_3d_batched_train instead of being recomputed."""
    cfg = d["cfg"]
    idx, w = M.moe_route_topk(d["logits"], cfg.k)
    gu = M.moe_gate_up_3d_batched_train(d["x"], d["w_gate_up"], idx, cfg.k)[1] if saved else None
    res = M.moe_backward_batched(d["x"], d["w_gate_up"], d["w_down"], idx, w, dout, cfg.k,
                                 gu_saved=gu)
    torch.cuda.synchronize()
    return res, idx


def _fp32(got, ref, bound, what):
    g = to_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    rl = rel_l2(g, ref) if np.any(ref != 0) else float(np.max(np.abs(g)))
    print(f"[parity] {what}: rel_l2={rl:.3e}", flush=True)
    assert rl <= bound, f"{what}: {rl:.3e} > {bound}"


def _check(M, d, what, tokens=None, experts=None, seed=0, saved=False):
    cfg = d["cfg"]
    print(f"[backward] {what}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} saved={saved}",
          flush=True)
    dout = W.make_output_grad(cfg, seed=seed, device="cuda")
    (dx, dwgu, dwd, dtw, dl), idx = run_bwd(M, d, dout, saved=saved)
    if isinstance(experts, int):                      # that many experts some token routes to:
        ii = idx.cpu().numpy()                        # the most- and least-loaded, then random
        used = np.unique(ii)
        cnt = np.bincount(ii.ravel(), minlength=cfg.E)
        rng = np.random.default_rng(7)
        ext = [int(used[np.argmax(cnt[used])]), int(used[np.argmin(cnt[used])])]
        rest = [int(e) for e in rng.permutation(used) if e not in ext]
        experts = np.array(sorted(set(ext + rest[:max(0, experts - 2)])), dtype=np.int64)
        print(f"[backward] experts {experts.tolist()} with {cnt[experts].tolist()} rows", flush=True)
    ref = oracle_backward(d, dout, tokens=tokens, experts=experts)
    ts = slice(None) if tokens is None else torch.as_tensor(tokens, device="cuda")
    es = slice(None) if experts is None else torch.as_tensor(experts, device="cuda")
    check_bf16(dx[ts], ref["dx"], what + " dx")
    check_bf16(dwgu[es], ref["dw_gate_up"], what + " dw_gate_up")
    check_bf16(dwd[es], ref["dw_down"], what + " dw_down")
    _fp32(dtw[ts], ref["d_topk_w"], DTW_REL_L2, what + " d_topk_w")
    _fp32(dl[ts], ref["dlogits"], DLOGITS_REL_L2, what + " dlogits")
    # experts outside each token's selection get exactly zero
    gl = to_f64(dl[ts])
    assert np.all(gl[ref["dlogits"] == 0.0] == 0.0) or cfg.k == 1
    if experts is None:                               # unrouted experts: zero weight gradients
        unused = sorted(set(range(cfg.E)) - set(np.unique(idx.cpu().numpy()).tolist()))
        for e in unused:
            assert not torch.any(dwgu[e].view(torch.int16)) and not torch.any(dwd[e].view(torch.int16))
    return dx, dwgu, dwd, dtw, dl


def _custom(T, H, I, E, k, seed=0):
    cfg = W.Config(name=f"bwd-T{T}-H{H}-I{I}-E{E}-k{k}", T=T, H=H, E=E, k=k, I=I, path="batched")
    return W.make(cfg, seed=seed, device="cuda")


@pytest.mark.parametrize("T,H,I,E,k", [
    (1, 256, 256, 4, 2),        # one token, two experts with one row each
    (100, 512, 256, 8, 2),      # ~25 rows per expert
    (300, 256, 512, 6, 3),      # ~150 rows per expert: several M-tiles, ragged K tail
    (257, 768, 256, 40, 8),     # many small experts, some empty
    (200, 512, 256, 5, 1),      # k = 1: dx written directly, no logit gradient
    (64, 256, 256, 16, 16),     # k = E
    (150, 1280, 768, 8, 2),     # 64-row tiles: dh over 3 and dx over 5 blocks of 256 columns
])
def test_backward_shapes(M, T, H, I, E, k):
    _check(M, _custom(T, H, I, E, k, seed=T + E), f"bwd T={T} k={k}")


@pytest.mark.parametrize("T,H,I,E,k", [
    (100, 512, 256, 8, 2),
    (300, 256, 512, 6, 3),
    (257, 768, 256, 40, 8),
    (200, 512, 256, 5, 1),
])
def test_backward_with_saved_preactivations(M, T, H, I, E, k):
    _check(M, _custom(T, H, I, E, k, seed=T + E + 1), f"bwd saved T={T} k={k}", saved=True)


def test_train_forward_matches_forward_and_oracle(M):
    # same h as the inference call (same kernel arithmetic), the same output after
    # the down projection, and FP32 pre-activations close to the oracle's
    d = _custom(300, 512, 256, 6, 3, seed=12)
    cfg = d["cfg"]
    idx, w = M.moe_route_topk(d["logits"], cfg.k)
    h0, _, ws0 = M.moe_gate_up_3d_batched(d["x"], d["w_gate_up"], idx, cfg.k)
    out0 = M.moe_down_3d_batched(h0, d["w_down"], idx, w, ws0, cfg.k)
    h1, gu, ws1 = M.moe_gate_up_3d_batched_train(d["x"], d["w_gate_up"], idx, cfg.k)
    out1 = M.moe_down_3d_batched(h1, d["w_down"], idx, w, ws1, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    from tests._gpu import oracle
    _, inter = oracle(d, return_intermediates=True)
    ref = inter["gu"].reshape(cfg.T * cfg.k, 2 * cfg.I)
    _fp32(gu, ref, 1e-5, "train forward gu")


@pytest.mark.parametrize("T,H,I,E,k", [
    (1100, 512, 256, 4, 1),     # large-group GEMMs, last round cut along K (fix-up epilogue)
    (600, 256, 512, 2, 2),      # k = 2, ragged last tile
])
def test_train_forward_large_groups(M, T, H, I, E, k):
    # >= 256 routed rows per expert: the large-group gate_up keeps the pre-activations
    # too, in its own epilogue and in the fix-up of the K-split tail
    d = _custom(T, H, I, E, k, seed=T + 3)
    cfg = d["cfg"]
    idx, w = M.moe_route_topk(d["logits"], cfg.k)
    h0, _, ws0 = M.moe_gate_up_3d_batched(d["x"], d["w_gate_up"], idx, cfg.k)
    h1, gu, ws1 = M.moe_gate_up_3d_batched_train(d["x"], d["w_gate_up"], idx, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    from tests._gpu import oracle
    _, inter = oracle(d, return_intermediates=True)
    ref = inter["gu"].reshape(cfg.T * cfg.k, 2 * cfg.I)
    _fp32(gu, ref, 1e-5, "train forward gu (large groups)")
    _check(M, d, f"bwd saved, large groups T={T} k={k}", saved=True)


def test_backward_large_groups_with_empty_expert(M):
    # >= 256 routed rows per expert on average: the weight gradients run on the
    # large-group GEMM over transposed, zero-padded operands; expert 3 gets no rows
    # (its gradients must be exactly zero) and the others ragged counts
    T, E = 1500, 4
    d = _custom(T, 256, 256, E, 2, seed=31)
    lg = d["logits"].clone()
    lg[:, 3] = -30.0
    d["logits"] = lg.contiguous()
    _check(M, d, "bwd large groups, one empty expert")
    _check(M, d, "bwd large groups, one empty expert, saved", saved=True)


def test_backward_large_groups_padded_grid(M):
    # E = 3 experts, H = I = 256: 6 dW_gate_up and 3 dW_down blocks of 256 x 256, so the
    # weight-gradient grids carry idle padding workgroups; k = 1 writes dx directly
    d = _custom(800, 256, 256, 3, 1, seed=41)
    _check(M, d, "bwd large groups, E = 3", saved=True)


def test_backward_bit_identical_repeats(M):
    d = _custom(600, 512, 256, 12, 4, seed=5)
    dout = W.make_output_grad(d["cfg"], seed=1, device="cuda")
    first, _ = run_bwd(M, d, dout)
    first = [t.clone() for t in first]
    for _ in range(3):
        again, _ = run_bwd(M, d, dout)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("saved", [False, True])
def test_backward_kimi_full_size(M, saved):
    d = W.make("kimi-bf16-T2048", seed=0, device="cuda")
    cfg = d["cfg"]
    toks, _ = sample_tokens(d["logits"].cpu().numpy(), cfg.k, 32, 2, n_focus=2)
    _check(M, d, f"kimi-bf16-T2048 ({toks.size} tokens, 8 experts)", tokens=toks, experts=8,
           saved=saved)


def test_backward_ep64_share_full_size(M):
    # ~2,700 rows per expert: long K loops in the weight gradients
    d = W.make("kimi-bf16-ep64share", seed=0, device="cuda")
    cfg = d["cfg"]
    toks, _ = sample_tokens(d["logits"].cpu().numpy(), cfg.k, 32, 3, n_focus=2)
    _check(M, d, f"kimi-bf16-ep64share ({toks.size} tokens, 3 experts)", tokens=toks, experts=3)
