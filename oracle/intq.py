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

The same formula block gives the asymmetric (zero-point) map:
s = (x_max - x_min) / (2**b - 1), z = round(-x_min / s),
q = clamp(round(x / s) + z, 0, 2**b - 1), x_hat = s * (q - z).
``asymmetric_quantize`` evaluates it in float64 over one group.
``int4g_asym_quantize`` is its per-group INT4 storage form, with these
readings:

* the range is widened to contain 0: lo = min(0, min w), hi = max(0, max w),
  so z is an integer in [0, 15] and 0 is represented exactly;
* s16 = fp16_RNE(fl32(fl32(hi - lo) / 15)); z = clamp(rint(fl32(-lo / s16)),
  0, 15); q = clamp(rint(fl32(w / s16)) + z, 0, 15); q = z = 0 where s16 == 0;
* q stored as unsigned nibbles (element 2j in bits 0-3 of byte j), s16 as
  fp16 [N, K/group], z as one uint8 per group [N, K/group].

Its GEMM is ``bf16_RNE(sum_k x[m,k] * s16[n, k/g] * (q[n,k] - z[n, k/g]))``
summed in float64.

Parity: pinned by tests/test_oracle_intq.py -- the page's worked INT8
example and outlier example (tests/golden/int8_worked_example.txt), a derived
INT4 example, the s/2 error bound, and a pure-Python triple loop; the
asymmetric forms by a hand-worked group
(tests/golden/int4_asym_worked_example.txt), the s/2 bound on unclamped
elements, a brute-force nearest-level search, exact zeros, and a triple loop.
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


def asymmetric_quantize(x, bits):
    """The page's asymmetric (zero-point) formula over one group, float64.

    Returns (s, z, q, x_hat); x_min / x_max are the group's extremes and
    round() is half-to-even.
    """
    x = np.asarray(x, dtype=np.float64)
    qmax = 2 ** bits - 1
    x_min, x_max = np.min(x), np.max(x)
    s = (x_max - x_min) / qmax
    if s == 0:
        return s, 0, np.zeros(x.shape, dtype=np.int64), np.zeros(x.shape)
    z = int(np.rint(-x_min / s))
    q = np.clip(np.rint(x / s) + z, 0, qmax).astype(np.int64)
    return s, z, q, s * (q - z)


INT4_ASYM_QMAX = 15


def int4g_asym_quantize(w, group=128):
    """Per-group asymmetric INT4 of a bf16 matrix W [N, K] (K % group == 0).

    Returns (packed uint8 [N, K/2], scales fp16 bit patterns uint16
    [N, K/group], zeros uint8 [N, K/group], q uint8 [N, K]).
    """
    w = np.asarray(w)
    wf = F.bf16_from_bits(w) if w.dtype == np.uint16 else w.astype(np.float32)
    if wf.ndim != 2 or wf.shape[1] % group:
        raise ValueError("int4g_asym_quantize expects [N, K] with K % group == 0")
    N, K = wf.shape
    grp = wf.reshape(N, K // group, group)
    lo = np.minimum(np.min(grp, axis=2), np.float32(0)).astype(np.float32)
    hi = np.maximum(np.max(grp, axis=2), np.float32(0)).astype(np.float32)
    span = (hi - lo).astype(np.float32)
    s32 = (span / np.float32(INT4_ASYM_QMAX)).astype(np.float32)
    s16 = F.fp16_round(s32).astype(np.float32)            # exact widening
    ok = s16 != 0
    safe = np.where(ok, s16, np.float32(1))
    z = np.where(ok, np.clip(np.rint((-lo / safe).astype(np.float32)), 0, INT4_ASYM_QMAX), 0)
    y = (grp / safe[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(y) + z[:, :, None], 0, INT4_ASYM_QMAX)
    q = np.where(ok[:, :, None], q, 0).astype(np.uint8).reshape(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, F.fp16_bits(s16.astype(np.float64)), z.astype(np.uint8), q


def int4_unpack_unsigned(packed):
    """uint8 [N, K/2] -> unsigned nibbles uint8 [N, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def int4g_asym_dequantize(packed, scales_bits, zeros, group=128):
    """s16 * (q - z) as float64 [N, K]."""
    q = int4_unpack_unsigned(packed).astype(np.float64)
    s = np.repeat(F.fp16_from_bits(scales_bits), group, axis=1)
    z = np.repeat(np.asarray(zeros, dtype=np.float64), group, axis=1)
    return s * (q - z)


def int4g_asym_gemm_fp64(x, packed, scales_bits, zeros, group=128):
    """Unrounded sum_k x[m,k] * s16 * (q - z) in float64, [M, N]."""
    x = np.asarray(x)
    xf = F.bf16_from_bits(x) if x.dtype == np.uint16 else x.astype(np.float32)
    return xf.astype(np.float64) @ int4g_asym_dequantize(packed, scales_bits, zeros, group).T


def int4g_asym_gemm(x, packed, scales_bits, zeros, group=128):
    """Y_ref = bf16_RNE(int4g_asym_gemm_fp64(...))."""
    return F.bf16_round(int4g_asym_gemm_fp64(x, packed, scales_bits, zeros, group))
