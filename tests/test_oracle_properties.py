"""Property tests of the oracle over random small shapes (hypothesis).

Each property follows from the definition of the layer, not from the oracle's
code: routing selects a top-k set with the lowest-index tie-break and weights
that sum to one; identical experts make the layer one dense SwiGLU FFN;
k = E makes it the softmax-weighted mixture of all experts; relabelling the
experts changes nothing; the layer is linear in W_down; every token's output
depends on that token alone; the MX encoding round-trips its own codes and
stays within half a step of its input.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import formats as F
from oracle import moe_forward, route

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@st.composite
def routing_case(draw):
    T = draw(st.integers(1, 6))
    E = draw(st.integers(1, 12))
    k = draw(st.integers(1, E))
    # logits on a coarse grid, so that ties (and +-0) are common
    vals = draw(st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0]),
                         min_size=T * E, max_size=T * E))
    return np.array(vals, dtype=np.float32).reshape(T, E), k


@SETTINGS
@given(routing_case())
def test_route_is_top_k_with_lowest_index_ties(case):
    logits, k = case
    idx, w = route(logits, k)
    T, E = logits.shape
    for t in range(T):
        sel = list(idx[t])
        assert len(set(sel)) == k
        rest = [e for e in range(E) if e not in sel]
        lo = min(float(logits[t, e]) for e in sel)
        for e in rest:                                  # nothing unselected is larger ...
            assert float(logits[t, e]) <= lo
            if float(logits[t, e]) == lo:               # ... and a tie goes to the lower index
                assert all(s < e for s in sel if float(logits[t, s]) == lo)
        # slots in (logit descending, index ascending) order
        keys = [(-float(logits[t, e]), e) for e in sel]
        assert keys == sorted(keys)
        assert abs(w[t].sum() - 1.0) <= 4 * k * 2.0 ** -53
        assert np.all(w[t] > 0) and np.all(np.diff(w[t]) <= 0)


@st.composite
def layer_case(draw, same_experts=False, k_all=False):
    T = draw(st.integers(1, 4))
    H = draw(st.sampled_from([2, 4, 8]))
    I = draw(st.sampled_from([1, 2, 4]))
    E = draw(st.integers(1, 5))
    k = E if k_all else draw(st.integers(1, E))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    x = _bf16_bits(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if same_experts:
        wgu = np.broadcast_to(_bf16_bits(rng.standard_normal((2 * I, H)) * 0.5), (E, 2 * I, H)).copy()
        wd = np.broadcast_to(_bf16_bits(rng.standard_normal((H, I)) * 0.5), (E, H, I)).copy()
    else:
        wgu = _bf16_bits(rng.standard_normal((E, 2 * I, H)) * 0.5)
        wd = _bf16_bits(rng.standard_normal((E, H, I)) * 0.5)
    return x, logits, wgu, wd, k


def _dense_ffn(x, wgu, wd):
    """SwiGLU FFN with torch float64 (a library silu, not the oracle's)."""
    xt = torch.from_numpy(F.bf16_decode(x))
    g = torch.from_numpy(F.bf16_decode(wgu))
    d = torch.from_numpy(F.bf16_decode(wd))
    I = g.shape[0] // 2
    a = torch.nn.functional.silu(xt @ g[:I].T) * (xt @ g[I:].T)
    return (a @ d.T).numpy()


@SETTINGS
@given(layer_case(same_experts=True))
def test_identical_experts_are_one_dense_ffn(case):
    x, logits, wgu, wd, k = case
    out = moe_forward(x, logits, wgu, wd, k)
    want = _dense_ffn(x, wgu[0], wd[0])
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12 * max(1.0, np.abs(want).max()))


@SETTINGS
@given(layer_case(k_all=True))
def test_k_equal_e_is_the_softmax_mixture(case):
    x, logits, wgu, wd, k = case
    out = moe_forward(x, logits, wgu, wd, k)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    want = sum(p[:, e:e + 1] * _dense_ffn(x, wgu[e], wd[e]) for e in range(wgu.shape[0]))
    assert np.allclose(out, want, rtol=1e-11, atol=1e-11 * max(1.0, np.abs(want).max()))


@SETTINGS
@given(layer_case(), st.integers(0, 2 ** 31 - 1))
def test_relabelling_experts_changes_nothing(case, pseed):
    x, logits, wgu, wd, k = case
    E = wgu.shape[0]
    perm = np.random.default_rng(pseed).permutation(E)
    # with distinct logits (N(0,1) draws) the slot order does not depend on labels
    out = moe_forward(x, logits, wgu, wd, k)
    out_p = moe_forward(x, logits[:, perm], wgu[perm], wd[perm], k)
    assert np.array_equal(out, out_p)


@SETTINGS
@given(layer_case(), st.integers(-3, 3))
def test_linear_in_w_down_and_tokens_independent(case, j):
    x, logits, wgu, wd, k = case
    out = moe_forward(x, logits, wgu, wd, k)
    wd2 = _bf16_bits(F.bf16_decode(wd) * 2.0 ** j)     # exact power-of-two scaling
    assert np.array_equal(moe_forward(x, logits, wgu, wd2, k), out * 2.0 ** j)
    T = x.shape[0]
    for t in range(T):          # (BLAS may block a one-row product differently: 1e-14)
        one = moe_forward(x, logits, wgu, wd, k, tokens=[t])[0]
        assert np.allclose(one, out[t], rtol=1e-14, atol=1e-14 * max(1e-300, np.abs(out[t]).max()))


@SETTINGS
@given(st.integers(1, 4), st.integers(1, 3), st.floats(1e-6, 1e6), st.integers(0, 2 ** 31 - 1))
def test_mx_quantize_round_trip_and_error_bound(rows, nblk, scale, seed):
    v = np.random.default_rng(seed).standard_normal((rows, 32 * nblk)) * scale
    codes, scales = F.mx_quantize(v)
    deq = F.mx_dequantize(codes, scales)
    c2, s2 = F.mx_quantize(deq)                       # a decoded block re-encodes to itself
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # in units of the block scale 2^s, every element is within half an E4M3 step
    # of its value (step 2^(floor(log2 |b|) - 3), or 2^-9 below 2^-6), except
    # that values above 448 saturate to 448
    s = scales.astype(np.int64) - 127
    blocks = v.reshape(rows, nblk, 32) / np.exp2(s)[..., None]
    err = np.abs(deq.reshape(rows, nblk, 32) / np.exp2(s)[..., None] - blocks)
    _, ex = np.frexp(np.abs(blocks))
    step = np.exp2(np.maximum(ex - 1, -6) - 3)        # E4M3 spacing at that magnitude
    assert np.all(err <= np.maximum(step / 2, np.abs(blocks) - 448.0))
    assert np.all(np.abs(blocks).max(axis=-1) < 512.0)   # the block max lands below 2^9
