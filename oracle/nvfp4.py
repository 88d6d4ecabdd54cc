"""NVFP4 quantization and the block-scaled 4-bit GEMM, as plain numpy.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix:

* "Tu pipeline NVFP4 ..." section 2 ("Qué es realmente NVFP4"): E2M1
  elements, blocks of 16 consecutive values sharing one scale, the scale
  stored as FP8 E4M3; the table in that section picks the scale from the
  block's largest magnitude ("absmax") and names 6 as the largest element.
* "NVFP4 en difusión ..." section 2 ("NVFP4 sin vLLM"): weights stored as a
  uint8 tensor (out, in/2) holding two FP4 values per byte, scales as a
  float8_e4m3fn tensor (out, in/16); the activation is quantized the same way
  on every forward; ``torch._scaled_mm(qact, qweight.t(), scale_a, scale_b,
  out_dtype=bfloat16)`` multiplies the decoded operands and emits bf16.

Readings taken where the pages are silent (each listed in the design notes):

1. A second-level per-tensor fp32 scale g = amax(|X|) / (6 * 448) is used for
   both operands (activations: one g over the whole [M, K] tensor per call).
   A caller may pass its own g instead.
2. Scale arithmetic is fp32 with one rounding per operation, in this order:
   s_raw = fl32(fl32(amax_b / 6) / g); s = E4M3_RNE_sat(s_raw);
   d = fl32(s * g); y = fl32(x / d).
3. Elements are divided by the *stored* (E4M3-rounded) scale times g.
4. E2M1 rounding is round-to-nearest with ties to the even code, saturating
   at 6.
5. The sign bit of x is kept, so a small negative value encodes as 0x8.
6. Element 2j goes to bits 0-3 of byte j, element 2j+1 to bits 4-7.
7. E4M3 is the OCP "fn" variant; values above 448 saturate to 448 (0x7E).
8. g == 0 or d == 0 gives magnitude 0 for every element of the block.
9. The GEMM sums in float64 and rounds the final value once to bf16.

Parity: pinned by tests/test_oracle_nvfp4.py -- a hand-worked three-block
row (tests/golden/nvfp4_worked_row.txt), the per-element error bound, a
pure-Python triple loop on tiny shapes, the unit-scale special case (plain
matmul of grid values), and W = diag(grid) reproducing dequant(A) exactly.
The weight-only product ``gemm_w4a16`` is pinned by a triple loop and by
equality with ``gemm`` when the bf16 activation is itself a dequantized
NVFP4 tensor with g = 1.
"""
import numpy as np

from . import formats as F

BLOCK = 16                       # values per scale block
E2M1_MAX = 6.0                   # largest E2M1 magnitude
GLOBAL_DENOM = np.float32(E2M1_MAX * F.E4M3_MAX)   # 2688, exact in fp32


def _as_bf16_values(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:                      # bf16 bit patterns
        return F.bf16_from_bits(x)
    x = x.astype(np.float32)
    F.bf16_bits(x)                                 # raises if not bf16-exact
    return x


def global_scale(x):
    """Per-tensor scale g = fl32(amax / 2688) of a bf16 tensor (fp32)."""
    xf = _as_bf16_values(x)
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    return np.float32(amax / GLOBAL_DENOM)


def quantize(x, g=None):
    """NVFP4-quantize a bf16 matrix X [R, C] (C % 16 == 0).

    ``x``: float32 array of bf16-exact values, or uint16 bf16 bit patterns.
    ``g``: optional per-tensor fp32 scale; computed from X when None.

    Returns (codes uint8 [R, C/2], scales uint8 [R, C/16] (E4M3 bytes),
    g float32).  Steps follow the order given in the module docstring.
    """
    xf = _as_bf16_values(x)
    if xf.ndim != 2 or xf.shape[1] % BLOCK:
        raise ValueError("quantize expects a 2-D array with C % 16 == 0")
    R, C = xf.shape
    g = global_scale(xf) if g is None else np.float32(g)

    blocks = xf.reshape(R, C // BLOCK, BLOCK)
    amax_b = np.max(np.abs(blocks), axis=2).astype(np.float32)     # exact
    if g == 0:
        s_raw = np.zeros_like(amax_b)
    else:
        s_raw = ((amax_b / np.float32(E2M1_MAX)).astype(np.float32) / g).astype(np.float32)
    s_code = F.e4m3_encode_nonneg(s_raw)                            # [R, C/16]
    s_val = F.e4m3_decode(s_code).astype(np.float32)                # exact
    d = (s_val * g).astype(np.float32)                              # fl32(s*g)

    d_b = np.broadcast_to(d[:, :, None], blocks.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(d_b != 0, blocks / np.where(d_b != 0, d_b, np.float32(1)), np.float32(0))
    y = y.astype(np.float32)                                        # fl32(x/d)
    mag = F.e2m1_encode_magnitude(np.abs(y))
    sign = np.signbit(blocks).astype(np.uint8)
    code = (sign << 3) | mag                                        # [R, C/16, 16]
    code = code.reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code.astype(np.uint8), np.float32(g)


def unpack_codes(packed):
    """uint8 [R, C/2] -> 4-bit codes [R, C] (low nibble = even element)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize_blockscaled(packed, scales):
    """value(code) * s per element, float64 [R, C] -- without g.

    This product has at most 6 significant bits and lies in [2**-10, 2688],
    so it is exact in bf16, fp16, fp32 and fp64.
    """
    codes = unpack_codes(packed)
    vals = F.e2m1_decode(codes)
    s = F.e4m3_decode(np.asarray(scales, dtype=np.uint8))
    return vals * np.repeat(s, BLOCK, axis=1)


def dequantize(packed, scales, g):
    """x_hat = value(code) * s * g, float64 [R, C]."""
    return dequantize_blockscaled(packed, scales) * np.float64(np.float32(g))


def gemm_fp64(a_codes, a_scales, a_g, w_codes, w_scales, w_g):
    """Unrounded fp64 result g_a * g_w * dequant(A) @ dequant(W)^T, [M, N]."""
    A = dequantize_blockscaled(a_codes, a_scales)
    W = dequantize_blockscaled(w_codes, w_scales)
    return (np.float64(np.float32(a_g)) * np.float64(np.float32(w_g))) * (A @ W.T)


def gemm(a_codes, a_scales, a_g, w_codes, w_scales, w_g):
    """Y_ref = bf16_RNE(g_a * g_w * sum_k A_hat[m,k] * W_hat[n,k]) in fp64.

    Returns float64 holding bf16 values, [M, N].
    """
    return F.bf16_round(gemm_fp64(a_codes, a_scales, a_g, w_codes, w_scales, w_g))


def gemm_w4a16_fp64(x, w_codes, w_scales, w_g):
    """Unrounded fp64 g_w * X @ dequant(W)^T with X a bf16 activation [M, K]
    (weight-only NVFP4: the activation is not quantized)."""
    X = _as_bf16_values(x).astype(np.float64)
    W = dequantize_blockscaled(w_codes, w_scales)
    return np.float64(np.float32(w_g)) * (X @ W.T)


def gemm_w4a16(x, w_codes, w_scales, w_g):
    """Y_ref = bf16_RNE(g_w * sum_k X[m,k] * W_hat[n,k]) in fp64, [M, N].

    The weight-only mode: "Cuantización e inferencia local" (section on
    activation outliers) notes that weight-only methods keep the activations
    in 16-bit; here the weight is NVFP4 exactly as for ``gemm`` and the
    activation stays bf16."""
    return F.bf16_round(gemm_w4a16_fp64(x, w_codes, w_scales, w_g))


def gemm_rows(a_codes, a_scales, a_g, w_codes, w_scales, w_g, rows):
    """``gemm`` restricted to the listed output rows (sampled parity at full
    sizes): the same definition, evaluated only where it is compared."""
    rows = np.asarray(rows)
    return gemm(np.asarray(a_codes)[rows], np.asarray(a_scales)[rows], a_g,
                w_codes, w_scales, w_g)
