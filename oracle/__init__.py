"""FP64 CPU oracle for the routed Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
package: only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline do.  It shares no code with the HIP path (its number-format codecs
are its own, written from the format definitions), and it is deliberately
plain and slow: NumPy float64, one expert at a time, no blocking or fusion.

Sources (the pages it follows):
  * warp-decode article (picklee.vercel.app, "Background" and "Key points"):
    expert routing, the two projection kernels gate_up and down, routed
    experts' contributions summed into FP32 accumulators, BF16 activations,
    no intermediate activation quantization;
  * Mixture-of-Kittens summary (asapai.co.kr, "What is 2.37x measured
    against"): MXFP8 and BF16 forward of the MoE layer; ("Determinism on par
    with performance"): a fixed floating-point order.
Readings taken where the pages are silent are listed in ``moe.py`` and in the
design notes of the repository.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against brute force, exact rational arithmetic, closed forms or library
routines, never against itself.
"""
from .formats import (bf16_decode, e4m3_decode, e4m3_encode, e8m0_decode,  # noqa: F401
                      mx_quantize, mx_dequantize, E4M3_MAX)
from .moe import route, silu, moe_forward  # noqa: F401
from .backward import moe_backward, moe_backward_mxfp8, silu_grad  # noqa: F401
