"""Python binding of libmoe_mi355x.so, the MI355X (gfx950) routed-MoE FFN library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The functions
carry the names of the C entry points in include/moe_mi355x.h; importing this
package raises ImportError when the library has not been built (there is no
fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_mi355x.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN = 0, -1, -2, -3
MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = -4, -5, -6
MOE_BF16, MOE_MXFP8 = 0, 1
KERNELS = {"none": 0, "route": 1, "decode_gate_up": 2, "decode_down": 3, "group": 4,
           "quant": 5, "gemm_gate_up": 6, "gemm_down": 7, "combine": 8, "bwd_gate_up": 9,
           "bwd_down": 10, "bwd_input": 11, "bwd_wdown": 12, "bwd_wgate_up": 13,
           "decode_fused": 14, "bwd_requant": 15}
MOE_DEBUG_PERMUTE_ORDER, MOE_DEBUG_DECODE_FUSED = 1, 2

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "moe_route_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_decode_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_decode_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_decode_forward_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_quantize_mxfp8": (_I, [_P, ctypes.c_int64, _I, _P, _P, _P]),
    "moe_gate_up_3d_batched": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "moe_down_3d_batched": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "moe_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_backward_batched": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                  _P, _P, _SZ, _P]),
    "moe_gate_up_3d_batched_train": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "moe_backward_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_backward_batched_mxfp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P,
                                        _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_backward_mxfp8_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_profile_kernel": (_I, [_I, _P, _P]),
    "moe_set_debug_options": (_I, [ctypes.c_uint, ctypes.c_uint32]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python mixture_experts_ffn_07_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        detail = lib.moe_last_error().decode()
        super().__init__(f"{fn}: {lib.moe_status_string(status).decode()} ({status}): {detail}")


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)   # 16-bit patterns read as BF16


def _u16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype not in _BF16:
        raise TypeError(f"expected BF16 bits, got {t.dtype}")
    return t


def _need(t: Optional[torch.Tensor], name: str, shape, dtypes, optional: bool = False) -> None:
    """Check a tensor argument's shape and element type before any pointer is
    handed to the library (a wrong size would become an out-of-bounds device
    access; a wrong dtype, e.g. int64 indices, would be misread)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_ws(ws: torch.Tensor, nbytes: int) -> None:
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} required")


def moe_route_topk(logits: torch.Tensor, k: int, topk_idx: torch.Tensor = None,
                   topk_w: torch.Tensor = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """logits [T, E] float32 -> (topk_idx [T, k] int32, topk_w [T, k] float32)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx),
                                                _ptr(topk_w), _stream(stream)))
    return topk_idx, topk_w


def moe_decode_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib.moe_decode_workspace_bytes(T, H, I, E, k))


def moe_workspace_bytes(T: int, H: int, I: int, E: int, k: int, dtype: int) -> int:
    return int(lib.moe_workspace_bytes(T, H, I, E, k, dtype))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device buffer for the workspace argument (256-byte aligned by torch)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def moe_decode_forward(x: torch.Tensor, logits: torch.Tensor, w_gate_up: torch.Tensor,
                       w_down: torch.Tensor, k: int, out: torch.Tensor = None,
                       topk_idx: torch.Tensor = None, topk_w: torch.Tensor = None,
                       ws: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Whole layer for a decode batch (T <= 64); BF16 in and out."""
    T, H = x.shape
    E, I2, H2 = w_gate_up.shape
    I = I2 // 2
    if logits.shape != (T, E) or H2 != H or tuple(w_down.shape) != (E, H, I):
        raise ValueError("inconsistent shapes")
    _u16(x), _u16(w_gate_up), _u16(w_down)
    _need(logits, "logits", (T, E), torch.float32)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", (T, H), _BF16)
    _need(topk_idx, "topk_idx", (T, k), torch.int32, optional=True)
    _need(topk_w, "topk_w", (T, k), torch.float32, optional=True)
    need = moe_decode_workspace_bytes(T, H, I, E, k)
    if ws is None:
        ws = workspace(need, x.device)
    _need_ws(ws, need)
    _check("moe_decode_forward", lib.moe_decode_forward(
        _ptr(x), _ptr(logits), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k, _ptr(out),
        _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))
    return out


STATIC_SCRATCH_BYTES = 4 << 20      # MOE_STATIC_SCRATCH_BYTES


def moe_decode_forward_noalloc(x: torch.Tensor, logits: torch.Tensor, w_gate_up: torch.Tensor,
                               w_down: torch.Tensor, k: int, out: torch.Tensor,
                               topk_idx: torch.Tensor = None, topk_w: torch.Tensor = None,
                               stream=None) -> torch.Tensor:
    """moe_decode_forward without a workspace (the library's own scratch); the
    caller passes every output, so this call allocates nothing."""
    T, H = x.shape
    E, I2, H2 = w_gate_up.shape
    I = I2 // 2
    if logits.shape != (T, E) or H2 != H or tuple(w_down.shape) != (E, H, I):
        raise ValueError("inconsistent shapes")
    _u16(x), _u16(w_gate_up), _u16(w_down)
    _need(logits, "logits", (T, E), torch.float32)
    _need(out, "out", (T, H), _BF16)
    _need(topk_idx, "topk_idx", (T, k), torch.int32, optional=True)
    _need(topk_w, "topk_w", (T, k), torch.float32, optional=True)
    _check("moe_decode_forward_noalloc", lib.moe_decode_forward_noalloc(
        _ptr(x), _ptr(logits), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k, _ptr(out),
        _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
    return out


def moe_quantize_mxfp8(src: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """src [rows, K] BF16 -> (E4M3 codes [rows, K] uint8, E8M0 scales [rows, K/32] uint8)."""
    rows, K = src.shape
    _u16(src)
    if codes is None:
        codes = torch.empty(rows, K, dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(rows, K // 32, dtype=torch.uint8, device=src.device)
    _need(codes, "codes", (rows, K), torch.uint8)
    _need(scales, "scales", (rows, K // 32), torch.uint8)
    _check("moe_quantize_mxfp8", lib.moe_quantize_mxfp8(_ptr(src), rows, K, _ptr(codes),
                                                        _ptr(scales), _stream(stream)))
    return codes, scales


def moe_gate_up_3d_batched(x, w_gate_up, topk_idx, k: int, dtype: int = MOE_BF16, x_scales=None,
                           w_gate_up_scales=None, h=None, h_scales=None, ws=None, stream=None):
    """Grouped gate/up projection + SwiGLU; returns (h, h_scales, ws)."""
    T, H = x.shape
    E, I2, H2 = w_gate_up.shape
    I = I2 // 2
    if H2 != H:
        raise ValueError("w_gate_up must be [E, 2I, H] with the H of x")
    mx = dtype == MOE_MXFP8
    edt = torch.uint8 if mx else _BF16
    _need(x, "x", (T, H), edt)
    _need(w_gate_up, "w_gate_up", (E, I2, H), edt)
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    if mx:
        _need(x_scales, "x_scales", (T, H // 32), torch.uint8)
        _need(w_gate_up_scales, "w_gate_up_scales", (E, I2, H // 32), torch.uint8)
    if h is None:
        h = torch.empty(T * k, I, dtype=torch.bfloat16 if dtype == MOE_BF16 else torch.uint8,
                        device=x.device)
    if mx and h_scales is None:
        h_scales = torch.empty(T * k, I // 32, dtype=torch.uint8, device=x.device)
    _need(h, "h", (T * k, I), edt)
    if mx:
        _need(h_scales, "h_scales", (T * k, I // 32), torch.uint8)
    need = moe_workspace_bytes(T, H, I, E, k, dtype)
    if ws is None:
        ws = workspace(need, x.device)
    _need_ws(ws, need)
    _check("moe_gate_up_3d_batched", lib.moe_gate_up_3d_batched(
        _ptr(x), _ptr(x_scales), _ptr(w_gate_up), _ptr(w_gate_up_scales), _ptr(topk_idx),
        T, H, I, E, k, dtype, _ptr(h), _ptr(h_scales), _ptr(ws), ws.numel(), _stream(stream)))
    return h, h_scales, ws


def moe_down_3d_batched(h, w_down, topk_idx, topk_w, ws, k: int, dtype: int = MOE_BF16,
                        h_scales=None, w_down_scales=None, out=None, stream=None):
    """Grouped down projection + fixed-order weighted combine -> out [T, H] BF16."""
    T = topk_idx.shape[0]
    E, H, I = w_down.shape
    mx = dtype == MOE_MXFP8
    edt = torch.uint8 if mx else _BF16
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _need(h, "h", (T * k, I), edt)
    _need(w_down, "w_down", (E, H, I), edt)
    if mx:
        _need(h_scales, "h_scales", (T * k, I // 32), torch.uint8)
        _need(w_down_scales, "w_down_scales", (E, H, I // 32), torch.uint8)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=h.device)
    _need(out, "out", (T, H), _BF16)
    _need_ws(ws, moe_workspace_bytes(T, H, I, E, k, dtype))
    _check("moe_down_3d_batched", lib.moe_down_3d_batched(
        _ptr(h), _ptr(h_scales), _ptr(w_down), _ptr(w_down_scales), _ptr(topk_idx),
        _ptr(topk_w), T, H, I, E, k, dtype, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_backward_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib.moe_backward_workspace_bytes(T, H, I, E, k))


def moe_gate_up_3d_batched_train(x, w_gate_up, topk_idx, k: int, h=None, gu=None, ws=None,
                                 stream=None):
    """moe_gate_up_3d_batched (BF16) that also returns the FP32 pre-activations;
    returns (h, gu, ws)."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _need(x, "x", (T, H), _BF16)
    _need(w_gate_up, "w_gate_up", (E, I2, H), _BF16)
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    if h is None:
        h = torch.empty(T * k, I, dtype=torch.bfloat16, device=x.device)
    if gu is None:
        gu = torch.empty(T * k, I2, dtype=torch.float32, device=x.device)
    _need(h, "h", (T * k, I), _BF16)
    _need(gu, "gu", (T * k, I2), torch.float32)
    need = moe_workspace_bytes(T, H, I, E, k, MOE_BF16)
    if ws is None:
        ws = workspace(need, x.device)
    _need_ws(ws, need)
    _check("moe_gate_up_3d_batched_train", lib.moe_gate_up_3d_batched_train(
        _ptr(x), _ptr(w_gate_up), _ptr(topk_idx), T, H, I, E, k, _ptr(h), _ptr(gu), _ptr(ws),
        ws.numel(), _stream(stream)))
    return h, gu, ws


def moe_backward_batched(x, w_gate_up, w_down, topk_idx, topk_w, dout, k: int, gu_saved=None,
                         dx=None, dw_gate_up=None, dw_down=None, d_topk_w=None, dlogits=None,
                         ws=None, stream=None):
    """Backward pass of the layer (BF16); returns (dx, dw_gate_up, dw_down, d_topk_w, dlogits)."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    dev = x.device
    _need(x, "x", (T, H), _BF16)
    _need(w_gate_up, "w_gate_up", (E, I2, H), _BF16)
    _need(w_down, "w_down", (E, H, I), _BF16)
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _need(dout, "dout", (T, H), _BF16)
    _need(gu_saved, "gu_saved", (T * k, I2), torch.float32, optional=True)
    if dx is None:
        dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if dw_gate_up is None:
        dw_gate_up = torch.empty(E, I2, H, dtype=torch.bfloat16, device=dev)
    if dw_down is None:
        dw_down = torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)
    if d_topk_w is None:
        d_topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    if dlogits is None:
        dlogits = torch.empty(T, E, dtype=torch.float32, device=dev)
    _need(dx, "dx", (T, H), _BF16)
    _need(dw_gate_up, "dw_gate_up", (E, I2, H), _BF16)
    _need(dw_down, "dw_down", (E, H, I), _BF16)
    _need(d_topk_w, "d_topk_w", (T, k), torch.float32)
    _need(dlogits, "dlogits", (T, E), torch.float32)
    need = moe_backward_workspace_bytes(T, H, I, E, k)
    if ws is None:
        ws = workspace(need, dev)
    _need_ws(ws, need)
    _check("moe_backward_batched", lib.moe_backward_batched(
        _ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(topk_idx), _ptr(topk_w), _ptr(dout),
        _ptr(gu_saved), T, H, I, E, k, _ptr(dx), _ptr(dw_gate_up), _ptr(dw_down), _ptr(d_topk_w), _ptr(dlogits),
        _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dw_gate_up, dw_down, d_topk_w, dlogits


def moe_set_debug_options(flags: int = 0, seed: int = 0) -> None:
    """Test options for this thread's later calls: MOE_DEBUG_PERMUTE_ORDER (permuted
    workgroup -> work-item order, seeded) and MOE_DEBUG_DECODE_FUSED (two-launch decode)."""
    _check("moe_set_debug_options", lib.moe_set_debug_options(int(flags), int(seed) & 0xFFFFFFFF))


def moe_backward_mxfp8_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib.moe_backward_mxfp8_workspace_bytes(T, H, I, E, k))


def moe_backward_batched_mxfp8(x, w_gate_up, w_gate_up_scales, w_down, w_down_scales, topk_idx,
                               topk_w, dout, k: int, dx=None, dw_gate_up=None, dw_down=None,
                               d_topk_w=None, dlogits=None, ws=None, stream=None):
    """Backward pass of the MXFP8 layer; returns (dx, dw_gate_up, dw_down, d_topk_w, dlogits)."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    dev = x.device
    _need(x, "x", (T, H), _BF16)
    _need(w_gate_up, "w_gate_up", (E, I2, H), torch.uint8)
    _need(w_gate_up_scales, "w_gate_up_scales", (E, I2, H // 32), torch.uint8)
    _need(w_down, "w_down", (E, H, I), torch.uint8)
    _need(w_down_scales, "w_down_scales", (E, H, I // 32), torch.uint8)
    _need(topk_idx, "topk_idx", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _need(dout, "dout", (T, H), _BF16)
    if dx is None:
        dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if dw_gate_up is None:
        dw_gate_up = torch.empty(E, I2, H, dtype=torch.bfloat16, device=dev)
    if dw_down is None:
        dw_down = torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)
    if d_topk_w is None:
        d_topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    if dlogits is None:
        dlogits = torch.empty(T, E, dtype=torch.float32, device=dev)
    _need(dx, "dx", (T, H), _BF16)
    _need(dw_gate_up, "dw_gate_up", (E, I2, H), _BF16)
    _need(dw_down, "dw_down", (E, H, I), _BF16)
    _need(d_topk_w, "d_topk_w", (T, k), torch.float32)
    _need(dlogits, "dlogits", (T, E), torch.float32)
    need = moe_backward_mxfp8_workspace_bytes(T, H, I, E, k)
    if ws is None:
        ws = workspace(need, dev)
    _need_ws(ws, need)
    _check("moe_backward_batched_mxfp8", lib.moe_backward_batched_mxfp8(
        _ptr(x), _ptr(w_gate_up), _ptr(w_gate_up_scales), _ptr(w_down), _ptr(w_down_scales),
        _ptr(topk_idx), _ptr(topk_w), _ptr(dout), T, H, I, E, k, _ptr(dx), _ptr(dw_gate_up),
        _ptr(dw_down), _ptr(d_topk_w), _ptr(dlogits), _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dw_gate_up, dw_down, d_topk_w, dlogits


def moe_profile_kernel(kernel, start_event: Optional[int], stop_event: Optional[int]) -> None:
    """Bracket the named kernel's launches with the given hipEvent_t handles."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check("moe_profile_kernel", lib.moe_profile_kernel(kid, start_event, stop_event))


__all__ = ["lib", "LIB_PATH", "MoeError", "moe_route_topk", "moe_decode_forward",
           "moe_decode_forward_noalloc", "STATIC_SCRATCH_BYTES",
           "moe_decode_workspace_bytes", "moe_workspace_bytes", "moe_quantize_mxfp8",
           "moe_gate_up_3d_batched", "moe_down_3d_batched", "moe_gate_up_3d_batched_train",
           "moe_backward_batched",
           "moe_backward_workspace_bytes", "moe_backward_batched_mxfp8",
           "moe_backward_mxfp8_workspace_bytes", "moe_profile_kernel", "workspace",
           "moe_set_debug_options", "MOE_DEBUG_PERMUTE_ORDER", "MOE_DEBUG_DECODE_FUSED",
           "MOE_BF16", "MOE_MXFP8", "KERNELS"]
