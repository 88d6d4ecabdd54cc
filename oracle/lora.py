"""Low-rank (LoRA) branch on an NVFP4 layer, as plain numpy.

Test infrastructure only (see ``oracle/__init__.py``).

What the page fixes ("NVFP4 en difusión ...", section 3, "¿Cómo
fine-tuneás algo que ya está en 4 bits?"): a low-rank correction cannot be
merged into NVFP4 weights -- they are discretized per block -- so it is
applied at run time, next to the quantized product, and the library the page
cites computes it in the same pass that quantizes the activation.

Readings taken where the page is silent (each listed in the design notes):

1. The layer computes y = g_a g_w A_hat W_hat^T + (X L_down^T) L_up^T, where
   X is the bf16 activation *before* quantization (the branch sees the
   high-precision input, read by the quantization pass), L_down is bf16
   [r, K] and L_up is bf16 [N, r] (both in the nn.Linear layout).  No extra
   scale factor (a LoRA alpha / r is folded into L_up by the caller).
2. The intermediate T = X L_down^T [M, r] is kept in fp32 on the device and
   in fp64 here; the output is rounded once to bf16.

Parity: pinned by tests/test_oracle_lora.py -- a pure-Python triple loop,
associativity (X L_down^T) L_up^T == X (L_up L_down)^T, and rank 0 (zero
factors) reducing to ``nvfp4.gemm``.
"""
import numpy as np

from . import formats as F
from . import nvfp4 as Q


def _bf16_values(a):
    a = np.asarray(a)
    return F.bf16_from_bits(a) if a.dtype == np.uint16 else a.astype(np.float32)


def lora_down(x, l_down):
    """T = X L_down^T in float64, [M, r]; X bf16 [M, K], L_down bf16 [r, K]."""
    return _bf16_values(x).astype(np.float64) @ _bf16_values(l_down).astype(np.float64).T


def gemm_lora_fp64(a_codes, a_scales, a_g, w_codes, w_scales, w_g, t, l_up):
    """Unrounded g_a g_w A_hat W_hat^T + T L_up^T in float64, [M, N]."""
    base = Q.gemm_fp64(a_codes, a_scales, a_g, w_codes, w_scales, w_g)
    return base + np.asarray(t, dtype=np.float64) @ _bf16_values(l_up).astype(np.float64).T


def gemm_lora(a_codes, a_scales, a_g, w_codes, w_scales, w_g, t, l_up):
    """Y_ref = bf16_RNE(gemm_lora_fp64(...)), float64 holding bf16 values."""
    return F.bf16_round(gemm_lora_fp64(a_codes, a_scales, a_g, w_codes, w_scales, w_g, t, l_up))
