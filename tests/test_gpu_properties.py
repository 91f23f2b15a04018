"""Random shapes within the documented limits against the FP64 oracle
(hypothesis, a fixed example sequence, a bounded number of examples per path).

Each example prints its shape before it runs, so a failure names its case."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as W
from oracle import route
from oracle.moe import rel_l2
from tests._gpu import MXFP8_REL_L2, check_bf16, oracle, to_f64

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=12, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(scope="module")
def M():
    import mixture_experts_ffn_07_amd as M
    return M


@st.composite
def shapes(draw, t_max, e_max, k_max):
    T = draw(st.integers(1, t_max))
    H = draw(st.sampled_from([256, 512, 768, 1024]))
    I = draw(st.sampled_from([256, 512, 768]))
    E = draw(st.integers(1, e_max))
    k = draw(st.integers(1, min(E, k_max)))
    seed = draw(st.integers(0, 10 ** 6))
    return T, H, I, E, k, seed


@SETTINGS
@given(shapes(64, 300, 16))
def test_decode_random_shapes(M, case):
    T, H, I, E, k, seed = case
    print(f"[property] decode T={T} H={H} I={I} E={E} k={k} seed={seed}", flush=True)
    cfg = W.Config(name="prop-dec", T=T, H=H, E=E, k=k, I=I)
    d = W.make(cfg, seed=seed, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    out = M.moe_decode_forward(d["x"], d["logits"], d["w_gate_up"], d["w_down"], k,
                               topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), route(d["logits"].cpu().numpy(), k)[0])
    check_bf16(out, oracle(d), f"decode T={T} H={H} I={I} E={E} k={k}")


@SETTINGS
@given(shapes(600, 48, 8), st.sampled_from(["bf16", "mxfp8"]))
def test_batched_random_shapes(M, case, dtype):
    T, H, I, E, k, seed = case
    print(f"[property] batched {dtype} T={T} H={H} I={I} E={E} k={k} seed={seed}", flush=True)
    cfg = W.Config(name="prop-bat", T=T, H=H, E=E, k=k, I=I, dtype=dtype, path="batched")
    d = W.make(cfg, seed=seed, device="cuda")
    idx, w = M.moe_route_topk(d["logits"], k)
    if dtype == "bf16":
        h, _, ws = M.moe_gate_up_3d_batched(d["x"], d["w_gate_up"], idx, k)
        out = M.moe_down_3d_batched(h, d["w_down"], idx, w, ws, k)
    else:
        xc, xs = M.moe_quantize_mxfp8(d["x"])
        h, hs, ws = M.moe_gate_up_3d_batched(xc, d["w_gate_up"], idx, k, M.MOE_MXFP8, x_scales=xs,
                                             w_gate_up_scales=d["w_gate_up_scales"])
        out = M.moe_down_3d_batched(h, d["w_down"], idx, w, ws, k, M.MOE_MXFP8, h_scales=hs,
                                    w_down_scales=d["w_down_scales"])
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), route(d["logits"].cpu().numpy(), k)[0])
    ref = oracle(d)
    what = f"batched {dtype} T={T} H={H} I={I} E={E} k={k}"
    if dtype == "bf16":
        check_bf16(out, ref, what)
    else:
        rl = rel_l2(to_f64(out), ref)
        print(f"[parity] {what}: rel_l2={rl:.3e}", flush=True)
        assert rl <= MXFP8_REL_L2
