"""Byte-equal results regardless of scheduling (Mixture-of-Kittens summary,
"Determinism on par with performance": the same output whatever order the
hardware runs the work in).

For every path (routing, decode at each batch-size regime and in its
single-launch form, batched BF16 at each tile height and on the large-group
GEMM with its K-split tail, MXFP8 small and large groups, MX quantization, the
backward on small and large groups): ten runs in the default order are byte
equal, and so are runs with the workgroup -> work-item order permuted by three
seeds (moe_set_debug_options(MOE_DEBUG_PERMUTE_ORDER, seed): a different
workgroup computes each item, in a different order)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

SEEDS = (1, 2, 3)


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    yield M
    M.moe_set_debug_options(0, 0)


def _bits(t):
    if t is None:
        return None
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.view(torch.int16).clone()
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).clone()
    return t.clone()


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        if x is None:
            continue
        assert torch.equal(x, y), f"{what}: output {i} differs"


def _check(M, run, what, flags=0):
    print(f"[determinism] {what}", flush=True)
    M.moe_set_debug_options(flags, 0)
    ref = [_bits(t) for t in run()]
    torch.cuda.synchronize()
    for _ in range(9):
        _same(ref, [_bits(t) for t in run()], f"{what} (repeat)")
    for s in SEEDS:
        M.moe_set_debug_options(flags | M.MOE_DEBUG_PERMUTE_ORDER, s)
        _same(ref, [_bits(t) for t in run()], f"{what} (permuted order, seed {s})")
    M.moe_set_debug_options(0, 0)


def _cfg(T, H, I, E, k, dtype="bf16", path="batched"):
    return W.Config(name=f"det-T{T}-H{H}-I{I}-E{E}-k{k}-{dtype}", T=T, H=H, E=E, k=k, I=I,
                    dtype=dtype, path=path)


@pytest.mark.parametrize("name,T", [("qwen3-decode-T1", 1), ("qwen3-decode-T8", 8),
                                    ("qwen3-decode-T32", 32), ("q35-zipf-T64", 64)])
def test_decode(M, name, T):
    d = W.make(name, seed=5, device="cuda")
    k = d["cfg"].k

    def run():
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        out = M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], k,
                                   topk_idx=idx, topk_w=w)
        return out, idx, w
    _check(M, run, f"decode {name}")
    if T <= 16:
        _check(M, run, f"decode {name}, single launch", flags=M.MOE_DEBUG_DECODE_FUSED)


def test_decode_wide_plain_loads(M):
    # T > 32 with H not a multiple of 512: the wide gate_up with plain loads
    d = W.make(_cfg(37, 768, 512, 40, 5, path="decode"), seed=6, device="cuda")

    def run():
        return (M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], 5),)
    _check(M, run, "decode T=37 H=768")


def test_route(M):
    g = torch.Generator(device="cuda").manual_seed(3)
    logits = torch.randn(3000, 384, generator=g, device="cuda")

    def run():
        return M.moe_route_topk(logits, 8)
    _check(M, run, "route 3000 x 384, k 8")


@pytest.mark.parametrize("T,H,I,E,k", [
    (2048, 512, 256, 64, 8),     # 64-row tiles, k > 1 (slot buffer + fixed-order combine)
    (700, 512, 256, 8, 2),       # 128-row tiles
    (1100, 512, 256, 4, 1),      # large-group GEMMs, K-split tail with its fix-up
    (600, 256, 512, 2, 2),       # large groups, k = 2
])
def test_batched_bf16(M, T, H, I, E, k):
    d = W.make(_cfg(T, H, I, E, k), seed=7, device="cuda")

    def run():
        idx, w = M.moe_route_topk(d["logits"], k)
        h, _, ws = M.moe_gate_up_3d_batched(d["x"], d["w_gate_up"], idx, k)
        out = M.moe_down_3d_batched(h, d["w_down"], idx, w, ws, k)
        return out, h, idx, w
    _check(M, run, f"batched BF16 T={T} E={E} k={k}")


@pytest.mark.parametrize("T,H,I,E,k", [
    (300, 512, 768, 6, 3),       # small groups
    (1100, 512, 256, 4, 1),      # large groups, K-split tail
])
def test_batched_mxfp8(M, T, H, I, E, k):
    d = W.make(_cfg(T, H, I, E, k, dtype="mxfp8"), seed=8, device="cuda")

    def run():
        idx, w = M.moe_route_topk(d["logits"], k)
        xc, xs = M.moe_quantize_mxfp8(d["x"])
        h, hs, ws = M.moe_gate_up_3d_batched(xc, d["w_gate_up"], idx, k, M.MOE_MXFP8, x_scales=xs,
                                             w_gate_up_scales=d["w_gate_up_scales"])
        out = M.moe_down_3d_batched(h, d["w_down"], idx, w, ws, k, M.MOE_MXFP8, h_scales=hs,
                                    w_down_scales=d["w_down_scales"])
        return out, h, hs, xc, xs
    _check(M, run, f"batched MXFP8 T={T} E={E} k={k}")


@pytest.mark.parametrize("T,H,I,E,k", [
    (600, 512, 256, 12, 4),      # small groups
    (1500, 256, 256, 4, 2),      # large groups: weight gradients, dx and dh on the large GEMM
])
def test_backward(M, T, H, I, E, k):
    d = W.make(_cfg(T, H, I, E, k), seed=9, device="cuda")
    dout = W.make_output_grad(d["cfg"], seed=1, device="cuda")

    def run():
        idx, w = M.moe_route_topk(d["logits"], k)
        _, gu, _ = M.moe_gate_up_3d_batched_train(d["x"], d["w_gate_up"], idx, k)
        res = M.moe_backward_batched(d["x"], d["w_gate_up"], d["w_down"], idx, w, dout, k,
                                     gu_saved=gu)
        return (gu,) + tuple(res)
    _check(M, run, f"backward T={T} E={E} k={k}")


@pytest.mark.parametrize("T,H,I,E,k", [
    (300, 256, 512, 6, 3),       # small groups, k > 1
    (1100, 512, 256, 4, 1),      # large groups, K-split tails
])
def test_backward_mxfp8(M, T, H, I, E, k):
    d = W.make(_cfg(T, H, I, E, k, dtype="mxfp8"), seed=10, device="cuda")
    dout = W.make_output_grad(d["cfg"], seed=2, device="cuda")

    def run():
        idx, w = M.moe_route_topk(d["logits"], k)
        return M.moe_backward_batched_mxfp8(d["x"], d["w_gate_up"], d["w_gate_up_scales"],
                                            d["w_down"], d["w_down_scales"], idx, w, dout, k)
    _check(M, run, f"backward MXFP8 T={T} E={E} k={k}")
