"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


@pytest.fixture(scope="module")
def m():
    # the build script by path: importing the package needs the built library
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moe_mi355x_build", os.path.join(ROOT, "mixture_experts_ffn_07_amd", "build.py"))
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)
    if not os.path.exists(B.LIB):
        B.build()
    import mixture_experts_ffn_07_amd as M
    alt = os.environ.get("MOE_ABI_TEST_LIB")
    if alt:     # a sanitizer build of the host code (tests/test_abi_sanitized.py)
        lib = ctypes.CDLL(alt)
        for name, (res, args) in M._SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        M.lib = lib
    return M


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(m):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(m.lib, n), n
        assert ctypes.cast(getattr(m.lib, n), ctypes.c_void_p).value


def test_status_strings(m):
    assert m.lib.moe_status_string(0) == b"ok"
    for s in range(-6, 0):
        assert m.lib.moe_status_string(s) not in (b"ok", b"unknown status")
    assert m.lib.moe_status_string(5) == b"unknown status"


FAKE = 0x10000        # a 16-byte aligned address that is never dereferenced


def _dec(m, T=4, H=512, I=256, E=8, k=2, x=FAKE, lg=FAKE, wgu=FAKE, wd=FAKE, out=FAKE,
         ws=FAKE, wsb=None):
    if wsb is None:
        wsb = m.lib.moe_decode_workspace_bytes(max(T, 1), H, I, E, k)
    return m.lib.moe_decode_forward(x, lg, wgu, wd, T, H, I, E, k, out, None, None, ws, wsb, None)


def test_decode_validation(m):
    assert _dec(m, x=None) == m.MOE_ERR_NULL
    assert _dec(m, out=None) == m.MOE_ERR_NULL
    assert _dec(m, k=0) == m.MOE_ERR_SHAPE
    assert _dec(m, k=9) == m.MOE_ERR_SHAPE                 # k > E
    assert _dec(m, E=40, k=33) == m.MOE_ERR_SHAPE          # k > 32
    assert _dec(m, E=1025, k=2) == m.MOE_ERR_SHAPE
    assert _dec(m, H=384) == m.MOE_ERR_SHAPE               # not a multiple of 256
    assert _dec(m, I=128) == m.MOE_ERR_SHAPE
    assert _dec(m, T=0) == m.MOE_ERR_SHAPE
    assert _dec(m, T=65, wsb=1 << 30) == m.MOE_ERR_UNSUPPORTED
    assert _dec(m, ws=None) == m.MOE_ERR_WORKSPACE
    need = m.lib.moe_decode_workspace_bytes(4, 512, 256, 8, 2)
    assert _dec(m, wsb=need - 1) == m.MOE_ERR_WORKSPACE
    assert _dec(m, x=FAKE + 2) == m.MOE_ERR_ALIGN
    assert _dec(m, ws=FAKE + 8) == m.MOE_ERR_ALIGN
    assert b"aligned" in m.lib.moe_last_error()


def test_workspace_sizes(m):
    assert m.lib.moe_decode_workspace_bytes(0, 512, 256, 8, 2) == 0
    assert m.lib.moe_decode_workspace_bytes(65, 512, 256, 8, 2) == 0
    a = m.lib.moe_decode_workspace_bytes(1, 2048, 768, 128, 8)
    b = m.lib.moe_decode_workspace_bytes(32, 2048, 768, 128, 8)
    assert 0 < a < b
    # the activation hand-off (a BF16 array of T*k*I) dominates
    assert b >= 32 * 8 * 768 * 2
    assert m.lib.moe_workspace_bytes(2048, 7168, 2048, 384, 8, 0) > 0
    assert m.lib.moe_workspace_bytes(2048, 7168, 2048, 384, 8, 7) == 0


def test_route_validation(m):
    r = m.lib.moe_route_topk
    assert r(FAKE, 4, 8, 0, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert r(FAKE, 4, 8, 9, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert r(FAKE, -1, 8, 2, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert r(None, 4, 8, 2, FAKE, FAKE, None) == m.MOE_ERR_NULL
    assert r(None, 0, 8, 2, None, None, None) == m.MOE_OK        # T = 0 enqueues nothing


def test_quant_validation(m):
    q = m.lib.moe_quantize_mxfp8
    assert q(FAKE, 4, 48, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert q(FAKE, -1, 64, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert q(None, 4, 64, FAKE, FAKE, None) == m.MOE_ERR_NULL
    assert q(FAKE, 4, 64, FAKE + 1, FAKE, None) == m.MOE_ERR_ALIGN
    assert q(None, 0, 64, None, None, None) == m.MOE_OK


def test_batched_validation(m):
    g = m.lib.moe_gate_up_3d_batched
    need = m.lib.moe_workspace_bytes(64, 256, 256, 8, 2, 0)
    args = dict(T=64, H=256, I=256, E=8, k=2, dt=0)

    def call(x=FAKE, xs=None, w=FAKE, ws_=None, idx=FAKE, h=FAKE, hs=None, ws=FAKE, wsb=need, **kw):
        a = dict(args, **kw)
        return g(x, xs, w, ws_, idx, a["T"], a["H"], a["I"], a["E"], a["k"], a["dt"], h, hs, ws,
                 wsb, None)
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(H=200) == m.MOE_ERR_SHAPE
    assert call(H=384) == m.MOE_ERR_SHAPE                  # not a multiple of 256
    assert call(I=128) == m.MOE_ERR_SHAPE                  # not a multiple of 256
    assert call(dt=3) == m.MOE_ERR_SHAPE
    assert call(wsb=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(h=FAKE + 4) == m.MOE_ERR_ALIGN
    assert call(dt=1, wsb=m.lib.moe_workspace_bytes(64, 256, 256, 8, 2, 1)) == m.MOE_ERR_NULL
    d = m.lib.moe_down_3d_batched
    assert d(FAKE, None, FAKE, None, FAKE, None, 64, 256, 256, 8, 2, 0, FAKE, FAKE, need,
             None) == m.MOE_ERR_NULL


def test_profile_hook_validation(m):
    assert m.lib.moe_profile_kernel(99, None, None) == m.MOE_ERR_SHAPE
    assert m.lib.moe_profile_kernel(2, None, None) == m.MOE_OK
    assert m.lib.moe_profile_kernel(0, None, None) == m.MOE_OK


def test_backward_validation(m):
    b = m.lib.moe_backward_batched
    need = m.lib.moe_backward_workspace_bytes(64, 256, 256, 8, 2)
    assert need > 0
    assert m.lib.moe_backward_workspace_bytes(0, 256, 256, 8, 2) == 0

    def call(x=FAKE, dout=FAKE, dx=FAKE, dwgu=FAKE, ws=FAKE, wsb=need, T=64, H=256, I=256, E=8,
             k=2):
        return b(x, FAKE, FAKE, FAKE, FAKE, dout, None, T, H, I, E, k, dx, dwgu, FAKE, FAKE, FAKE,
                 ws, wsb, None)
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(dout=None) == m.MOE_ERR_NULL
    assert call(dwgu=None) == m.MOE_ERR_NULL
    assert call(H=384) == m.MOE_ERR_SHAPE
    assert call(I=128) == m.MOE_ERR_SHAPE
    assert call(T=0) == m.MOE_ERR_SHAPE
    assert call(k=9) == m.MOE_ERR_SHAPE
    assert call(ws=None) == m.MOE_ERR_WORKSPACE
    assert call(wsb=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(dx=FAKE + 2) == m.MOE_ERR_ALIGN
    # the workspace holds the recomputed FP32 pre-activations and the BF16 gradients
    # of [g; u] for every routed pair
    assert need >= 64 * 2 * 2 * 256 * (4 + 2)


def test_backward_mxfp8_validation(m):
    b = m.lib.moe_backward_batched_mxfp8
    need = m.lib.moe_backward_mxfp8_workspace_bytes(64, 256, 256, 8, 2)
    assert need > 0
    assert m.lib.moe_backward_mxfp8_workspace_bytes(0, 256, 256, 8, 2) == 0

    def call(x=FAKE, wgus=FAKE, wds=FAKE, dout=FAKE, dx=FAKE, dl=FAKE, ws=FAKE, wsb=need, T=64,
             H=256, I=256, E=8, k=2):
        return b(x, FAKE, wgus, FAKE, wds, FAKE, FAKE, dout, T, H, I, E, k, dx, FAKE, FAKE, FAKE,
                 dl, ws, wsb, None)
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(wgus=None) == m.MOE_ERR_NULL
    assert call(wds=None) == m.MOE_ERR_NULL
    assert call(dout=None) == m.MOE_ERR_NULL
    assert call(dl=None) == m.MOE_ERR_NULL
    assert call(H=384) == m.MOE_ERR_SHAPE
    assert call(I=128) == m.MOE_ERR_SHAPE
    assert call(T=0) == m.MOE_ERR_SHAPE
    assert call(k=9) == m.MOE_ERR_SHAPE
    assert call(ws=None) == m.MOE_ERR_WORKSPACE
    assert call(wsb=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(dx=FAKE + 2) == m.MOE_ERR_ALIGN
    assert call(wgus=FAKE + 8) == m.MOE_ERR_ALIGN
    # pair-axis operands: max(H, 2I) * (T*k + 128*E) must stay below 2^31
    big = 1 << 60
    assert call(T=149500, H=7168, I=256, k=2, wsb=big) == m.MOE_ERR_SHAPE   # T*k*H < 2^31
    assert b"max(H, 2I)" in m.lib.moe_last_error()
    # the workspace holds both weights re-encoded along their output axis
    wbytes = 8 * (2 * 256 * 256 + 256 * 256)
    assert need >= wbytes + wbytes // 32


def test_train_forward_validation(m):
    g = m.lib.moe_gate_up_3d_batched_train
    need = m.lib.moe_workspace_bytes(64, 256, 256, 8, 2, 0)

    def call(x=FAKE, gu=FAKE, T=64, H=256, I=256, E=8, k=2, wsb=need):
        return g(x, FAKE, FAKE, T, H, I, E, k, FAKE, gu, FAKE, wsb, None)
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(gu=None) == m.MOE_ERR_NULL
    assert call(I=128) == m.MOE_ERR_SHAPE
    assert call(wsb=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(gu=FAKE + 4) == m.MOE_ERR_ALIGN
    # T*k*2I must stay below 2^31 (pair-row offsets of gu are 32-bit)
    huge = m.lib.moe_workspace_bytes(1 << 20, 256, 1024, 8, 1, 0)
    assert call(T=1 << 20, I=1024, k=1, wsb=huge) == m.MOE_ERR_SHAPE


def test_batched_offset_limits(m):
    # the kernels form 32-bit element offsets: T*H, T*k*H, T*k*I and 2I*H must stay
    # below 2^31 (checked before the workspace, so any size passes here)
    g = m.lib.moe_gate_up_3d_batched
    d = m.lib.moe_down_3d_batched
    big = 1 << 60

    def gate_up(T, H, I, E, k):
        return g(FAKE, None, FAKE, None, FAKE, T, H, I, E, k, 0, FAKE, None, FAKE, big, None)

    def down(T, H, I, E, k):
        return d(FAKE, None, FAKE, None, FAKE, FAKE, T, H, I, E, k, 0, FAKE, FAKE, big, None)
    for call in (gate_up, down):
        assert call(300000, 7168, 256, 8, 1) == m.MOE_ERR_SHAPE            # T*H
        assert b"T*H" in m.lib.moe_last_error()
        assert call(1 << 18, 1024, 256, 8, 8) == m.MOE_ERR_SHAPE           # T*k*H = 2^31
        assert b"T*k*H" in m.lib.moe_last_error()
        assert call(1 << 18, 256, 1024, 8, 8) == m.MOE_ERR_SHAPE           # T*k*I = 2^31
        assert b"T*k*I" in m.lib.moe_last_error()
        assert call(4, 1 << 16, 1 << 14, 8, 2) == m.MOE_ERR_SHAPE          # 2*I*H = 2^31
        assert b"2*I*H" in m.lib.moe_last_error()
    # just below the limits the shape checks pass (here a misaligned h is next)
    assert g(FAKE, None, FAKE, None, FAKE, 4, 1 << 16, (1 << 14) - 256, 8, 2, 0, FAKE + 4, None,
             FAKE, big, None) == m.MOE_ERR_ALIGN
    assert g(FAKE, None, FAKE, None, FAKE, (1 << 18) - 1, 1024, 256, 8, 8, 0, FAKE + 4, None,
             FAKE, big, None) == m.MOE_ERR_ALIGN
    # decode: one expert's weights, 2*I*H, must stay below 2^31
    assert _dec(m, H=1 << 19, I=2048, wsb=big) == m.MOE_ERR_SHAPE
    assert b"2*I*H" in m.lib.moe_last_error()


def test_binding_validates_tensor_arguments(m):
    # the Python wrappers check shapes and dtypes before any pointer reaches the
    # library (CPU tensors of the right shape fail only at the device check)
    import torch
    T, H, I, E, k = 4, 256, 256, 8, 2
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    wgu = torch.zeros(E, 2 * I, H, dtype=torch.bfloat16)
    wd = torch.zeros(E, H, I, dtype=torch.bfloat16)
    logits = torch.zeros(T, E)
    idx = torch.zeros(T, k, dtype=torch.int32)
    tw = torch.zeros(T, k)
    with pytest.raises(TypeError, match="topk_idx"):
        m.moe_route_topk(logits, k, topk_idx=torch.zeros(T, k, dtype=torch.int64))
    with pytest.raises(ValueError, match="topk_w"):
        m.moe_route_topk(logits, k, topk_w=torch.zeros(T, k + 1))
    with pytest.raises(ValueError, match="GPU"):
        m.moe_route_topk(logits, k, topk_idx=idx, topk_w=tw)
    with pytest.raises(TypeError, match="topk_idx"):
        m.moe_gate_up_3d_batched(x, wgu, idx.long(), k, h=torch.zeros(T * k, I, dtype=torch.bfloat16),
                                 ws=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="h: shape"):
        m.moe_gate_up_3d_batched(x, wgu, idx, k, h=torch.zeros(T * k - 1, I, dtype=torch.bfloat16),
                                 ws=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="x_scales"):
        m.moe_gate_up_3d_batched(x.view(torch.uint8)[:, :H], wgu.view(torch.uint8)[..., :H], idx, k,
                                 m.MOE_MXFP8, x_scales=torch.zeros(T, H // 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        m.moe_gate_up_3d_batched(x, wgu, idx, k, h=torch.zeros(T * k, I, dtype=torch.bfloat16),
                                 ws=torch.zeros(16, dtype=torch.uint8))
    ws = torch.zeros(m.moe_workspace_bytes(T, H, I, E, k, m.MOE_BF16), dtype=torch.uint8)
    h = torch.zeros(T * k, I, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out: shape"):
        m.moe_down_3d_batched(h, wd, idx, tw, ws, k, out=torch.zeros(T, H + 1, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="topk_w"):
        m.moe_down_3d_batched(h, wd, idx, tw.double(), ws, k)
    with pytest.raises(ValueError, match="GPU"):
        m.moe_down_3d_batched(h, wd, idx, tw, ws, k)
    with pytest.raises(ValueError, match="codes"):
        m.moe_quantize_mxfp8(x, codes=torch.zeros(T, H - 32, dtype=torch.uint8))
    with pytest.raises(TypeError, match="topk_idx"):
        m.moe_decode_forward(x, logits, wgu, wd, k, topk_idx=tw)
    with pytest.raises(ValueError, match="gu_saved"):
        m.moe_backward_batched(x, wgu, wd, idx, tw, x, k, gu_saved=torch.zeros(T * k, I))


def test_debug_options_validation(m):
    assert m.lib.moe_set_debug_options(0, 0) == m.MOE_OK
    assert m.lib.moe_set_debug_options(m.MOE_DEBUG_PERMUTE_ORDER | m.MOE_DEBUG_DECODE_FUSED, 7) == m.MOE_OK
    assert m.lib.moe_set_debug_options(4, 0) == m.MOE_ERR_SHAPE
    assert b"unknown" in m.lib.moe_last_error()
    assert m.lib.moe_set_debug_options(0, 0) == m.MOE_OK
