"""Symmetric integer quantization (the general formula and its INT4
per-group weight-only form), as plain numpy.

Test infrastructure only (see ``oracle/__init__.py``).

Source: "Cuantización e inferencia local" (class 085 of the AI-evolution
course), the formula block: for b-bit symmetric quantization the scale is
s = max|x| / (2**(b-1) - 1), codes q = clamp(round(x / s), -(2**(b-1)-1),
2**(b-1)-1) and the reconstruction is s * q; the rounding error per element
is at most s/2; the scale is kept per group (per row, channel, or block of
32-128 weights) so one large weight does not ruin the rest.  The same page's
worked INT8 example and its outlier variant pin ``symmetric_quantize``.  The
"INT4 por-grupo" scheme also appears in the course plan "Fase 26 --
Inmersión en cuantización", section "Objetivo".

``symmetric_quantize`` evaluates the page's formula in float64 (the page
fixes no precision).  ``int4g_quantize`` is the per-group INT4 form used by
the W4A16 path, with the precision and storage the readings fix:

* groups of 128 consecutive values along K in each row;
* s16 = fp16_RNE(fl32(max|w_group| / 7)) (fp16 storage of the scale);
* q = clamp(rint_half_even(fl32(w / fl32(s16))), -7, 7), q = 0 where s16 == 0
  (the stored, rounded scale divides, so the reconstruction is consistent);
* each q stored as a two's-complement nibble, element 2j in bits 0-3 of byte
  j, element 2j+1 in bits 4-7.

The INT4 GEMM is ``bf16_RNE(sum_k x[m,k] * s16[n, k/128] * q[n,k])`` summed
in float64.

Parity: pinned by tests/test_oracle_intq.py -- the page's worked INT8
example and outlier example (tests/golden/int8_worked_example.txt), a derived
INT4 example, the s/2 error bound, and a pure-Python triple loop.
"""
import numpy as np

from . import formats as F


def symmetric_quantize(x, bits):
    """The page's symmetric formula over one group, in float64.

    Returns (s, q, x_hat) with q an int64 array; round() is half-to-even.
    """
    x = np.asarray(x, dtype=np.float64)
    qmax = 2 ** (bits - 1) - 1
    s = np.max(np.abs(x)) / qmax
    if s == 0:
        q = np.zeros(x.shape, dtype=np.int64)
    else:
        q = np.clip(np.rint(x / s), -qmax, qmax).astype(np.int64)
    return s, q, s * q


INT4_QMAX = 7


def int4g_quantize(w, group=128):
    """Per-group symmetric INT4 of a bf16 matrix W [N, K] (K % group == 0).

    ``w``: float32 bf16-exact values or uint16 bf16 bits.
    Returns (packed uint8 [N, K/2], scales fp16 bit patterns uint16
    [N, K/group], q int8 [N, K]).
    """
    w = np.asarray(w)
    wf = F.bf16_from_bits(w) if w.dtype == np.uint16 else w.astype(np.float32)
    if wf.ndim != 2 or wf.shape[1] % group:
        raise ValueError("int4g_quantize expects [N, K] with K % group == 0")
    N, K = wf.shape
    grp = wf.reshape(N, K // group, group)
    amax = np.max(np.abs(grp), axis=2).astype(np.float32)
    s32 = (amax / np.float32(INT4_QMAX)).astype(np.float32)
    s16 = F.fp16_round(s32)                            # float64 holding fp16
    s16_32 = s16.astype(np.float32)                    # exact widening
    den = np.broadcast_to(s16_32[:, :, None], grp.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(den != 0, grp / np.where(den != 0, den, np.float32(1)), np.float32(0))
    y = y.astype(np.float32)
    q = np.clip(np.rint(y), -INT4_QMAX, INT4_QMAX).astype(np.int8).reshape(N, K)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, F.fp16_bits(s16), q


def int4_unpack(packed):
    """uint8 [N, K/2] -> signed int8 [N, K] from two's-complement nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int16)
    nib[:, 0::2] = p & 0xF
    nib[:, 1::2] = p >> 4
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def int4g_dequantize(packed, scales_bits, group=128):
    """s16 * q as float64 [N, K]."""
    q = int4_unpack(packed).astype(np.float64)
    s = F.fp16_from_bits(scales_bits)
    return q * np.repeat(s, group, axis=1)


def int4g_gemm_fp64(x, packed, scales_bits, group=128):
    """Unrounded sum_k x[m,k] * s16[n,k/group] * q[n,k] in float64, [M, N]."""
    x = np.asarray(x)
    xf = F.bf16_from_bits(x) if x.dtype == np.uint16 else x.astype(np.float32)
    W = int4g_dequantize(packed, scales_bits, group)
    return xf.astype(np.float64) @ W.T


def int4g_gemm(x, packed, scales_bits, group=128):
    """Y_ref = bf16_RNE(int4g_gemm_fp64(...)), float64 holding bf16 values."""
    return F.bf16_round(int4g_gemm_fp64(x, packed, scales_bits, group))
