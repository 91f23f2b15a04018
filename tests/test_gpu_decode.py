"""GPU parity of the decode path (moe_decode_forward) against the FP64 oracle.

Every case prints its name and shape before running so that a failure names it."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import route
from tests._gpu import W_ABS, check_bf16, oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


def _run(M, d):
    cfg = d["cfg"]
    T = cfg.T
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    out = M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], cfg.k,
                               topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return out, idx, w


def _full_check(M, d, what):
    cfg = d["cfg"]
    print(f"[decode] {what}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    out, idx, w = _run(M, d)
    ridx, rw = route(d["logits"].cpu().numpy(), cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ridx), f"{what}: top-k indices differ"
    assert np.max(np.abs(w.cpu().double().numpy() - rw)) <= W_ABS
    ref = oracle(d)
    return check_bf16(out, ref, what), out


@pytest.mark.parametrize("name", ["tiny-T4", "qwen3-decode-T1", "qwen3-decode-T8",
                                  "qwen3-decode-T32", "q35-zipf-T64"])
def test_decode_workloads(M, name):
    d = W.make(name, seed=0, device="cuda")
    _full_check(M, d, name)


def _custom(T, H, I, E, k, seed=0, x_std=1.0):
    cfg = W.Config(name=f"custom-T{T}-H{H}-I{I}-E{E}-k{k}", T=T, H=H, E=E, k=k, I=I, x_std=x_std)
    return W.make(cfg, seed=seed, device="cuda")


@pytest.mark.parametrize("T,H,I,E,k", [
    (1, 256, 256, 4, 1),       # smallest sizes, k = 1 (weight exactly 1)
    (17, 512, 256, 8, 8),      # k = E: every expert, ragged second token tile
    (37, 768, 512, 40, 5),     # odd sizes, three token tiles
    (64, 256, 512, 1000, 32),  # k = 32, E near the limit
    (5, 1024, 2048, 16, 3),    # I = 2048: eight K-slices of 256 in down
    (48, 1024, 512, 24, 6),    # T > 32 with H % 512 == 0: whole-line gate_up, two steps per wave
    (3, 512, 1280, 8, 2),      # I = 1280: four K-slices of 320 in down
    (9, 256, 1792, 12, 3),     # I = 1792: four K-slices of 448 in down
])
def test_decode_shapes(M, T, H, I, E, k):
    _full_check(M, _custom(T, H, I, E, k, seed=T), f"shape T={T} H={H} I={I} E={E} k={k}")


def test_decode_all_tokens_one_expert_set(M):
    # identical logits rows: every token routes to the same k experts, so one
    # expert serves all 64 tokens (four full token tiles)
    d = _custom(64, 512, 256, 16, 4, seed=3)
    d["logits"] = d["logits"][:1].repeat(64, 1).contiguous()
    _full_check(M, d, "64 tokens on the same experts")


def test_decode_tied_logits(M):
    d = _custom(9, 256, 256, 12, 4, seed=4)
    d["logits"] = torch.zeros_like(d["logits"])
    d["logits"][3, 7] = -0.0
    _full_check(M, d, "all-zero logits")


def test_decode_reads_only_routed_experts(M):
    # poison every expert no token routes to: NaN would reach the output if read
    d = _custom(3, 512, 256, 32, 2, seed=5)
    ridx, _ = route(d["logits"].cpu().numpy(), 2)
    unused = sorted(set(range(32)) - set(ridx.ravel().tolist()))
    assert unused
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    d["w_gate_up"][unused] = nan.cuda()
    d["w_down"][unused] = nan.cuda()
    out, _, _ = _run(M, d)
    assert torch.isfinite(out.float()).all()


def test_decode_bit_identical_repeats(M):
    d = W.make("qwen3-decode-T32", seed=1, device="cuda")
    first, idx0, w0 = _run(M, d)
    for _ in range(5):
        out, idx, w = _run(M, d)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
        assert torch.equal(idx, idx0) and torch.equal(w.view(torch.int32), w0.view(torch.int32))


def test_decode_on_side_stream_and_null_outputs(M):
    d = W.make("tiny-T4", seed=2, device="cuda")
    ref, _, _ = _run(M, d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], 2)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_decode_rejects_large_batch(M):
    d = _custom(65, 256, 256, 4, 2)
    with pytest.raises(M.MoeError) as e:
        M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], 2)
    assert e.value.status == -5


def test_decode_accuracy_study(M):
    # the GPU decode (BF16 hand-off) against the FP64 oracle, beside the oracle's
    # own BF16-hand-off and FP8-hand-off variants (tests/test_accuracy_study.py)
    from oracle import moe_forward
    from oracle.formats import bf16_round
    from oracle.moe import rel_l2
    from tests._gpu import Fetch, bits
    d = W.make("qwen3-decode-T8", seed=0, device="cuda")
    cfg = d["cfg"]
    print(f"[decode] accuracy study: qwen3-decode-T8", flush=True)
    out, _, _ = _run(M, d)
    args = (bits(d["x"]), d["logits"].cpu().numpy(), Fetch(d["w_gate_up"]), Fetch(d["w_down"]), cfg.k)
    exact = moe_forward(*args)
    d_gpu = rel_l2(out.cpu().double().numpy(), exact)
    d_bf16 = rel_l2(bf16_round(moe_forward(*args, h_round="bf16")), exact)
    d_fp8 = rel_l2(bf16_round(moe_forward(*args, h_round="mxfp8")), exact)
    print(f"[accuracy] GPU decode {d_gpu:.3e}; oracle with BF16 h {d_bf16:.3e}, with MXFP8 h "
          f"{d_fp8:.3e}; FP8 / GPU = {d_fp8 / d_gpu:.2f}", flush=True)
    assert d_gpu < 1.2 * d_bf16
    assert d_fp8 > 3 * d_gpu


def _run_opts(M, d, flags):
    M.moe_set_debug_options(flags, 0)
    try:
        return _run(M, d)
    finally:
        M.moe_set_debug_options(0, 0)


@pytest.mark.parametrize("T,H,I,E,k", [
    (1, 2048, 768, 128, 8),     # the Qwen3-style shape at T = 1 (one down task per wave)
    (8, 2048, 768, 128, 8),     # T = 8: ~52 touched experts, tasks beyond the prefetched two
    (16, 2048, 768, 128, 8),    # T = 16: two token tiles, 16-neuron items
    (2, 7168, 512, 16, 2),      # 896 output groups: workgroups take several groups
    (4, 256, 256, 8, 2),        # 32 output groups: most workgroups have none
    (3, 512, 1536, 10, 3),      # I = 1536: eight K-slices of three steps
    (5, 1024, 2048, 16, 3),     # I = 2048: eight K-slices of four steps
])
def test_decode_single_launch_matches_two_launches(M, T, H, I, E, k):
    # T <= 16 runs as two launches by default; the debug option runs routing,
    # gate_up and down as one launch.  Both meet the oracle's bars, and agree
    # closely (the single launch's down phase sums its waves' partials in a
    # different fixed grouping)
    d = _custom(T, H, I, E, k, seed=100 + T)
    what = f"T={T} H={H} I={I} E={E} k={k}"
    print(f"[decode] single launch vs two launches {what}", flush=True)
    one, idx1, w1 = _run_opts(M, d, M.MOE_DEBUG_DECODE_FUSED)
    two, idx2, w2 = _run(M, d)
    assert torch.equal(idx1, idx2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    ref = oracle(d)
    check_bf16(one, ref, f"single launch {what}")
    check_bf16(two, ref, f"two launches {what}")
    from oracle.moe import rel_l2
    assert rel_l2(one.double().cpu().numpy(), two.double().cpu().numpy()) < 2e-3
    for _ in range(9):                                # ten byte-equal runs of the single launch
        again, _, _ = _run_opts(M, d, M.MOE_DEBUG_DECODE_FUSED)
        assert torch.equal(again.view(torch.int16), one.view(torch.int16))
