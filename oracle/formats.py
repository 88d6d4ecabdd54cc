"""Number formats used by NVFP4, written from their bit definitions.

Test infrastructure only (see ``oracle/__init__.py``).

Sources (the pages are cited by title and section):

* "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de laptop", section
  "2. Qué es realmente NVFP4": each element is E2M1 (1 sign bit, 2 exponent
  bits, 1 mantissa bit); 16 consecutive values share one scale stored as FP8
  with 4 exponent and 3 mantissa bits (E4M3); the "four-over-six" row of the
  scale-selection table names 6 as the largest element magnitude.
* "NVFP4 en difusión: la misma cuantización, un motor completamente
  distinto", section "2. NVFP4 sin vLLM: torch._scaled_mm a mano": the scale
  dtype is ``float8_e4m3fn`` (the OCP "finite" FP8 variant: no infinities,
  only 0x7F/0xFF are NaN, largest finite value 448) and the product is
  emitted as bfloat16.

Parity: every function here is pinned (tests/test_oracle_formats.py):
E2M1 decode by the closed-form derivation of its grid, E2M1 encode by a
brute-force nearest-grid search, E4M3 decode/encode by torch's CPU
``float8_e4m3fn`` cast, bf16 / fp16 rounding by torch's CPU casts and a
brute-force two-candidate search.
"""
import numpy as np

# ---------------------------------------------------------------- E2M1 ----
# Bit layout s|e1 e0|m.  With 2 exponent bits the largest magnitude is 6 only
# with an exponent bias of 1:  (1 + 1/2) * 2**(3 - 1) = 6.  Exponent field 0
# is subnormal: m * 2**(1 - 1) * 1/2.
E2M1_BIAS = 1


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code (array of ints 0..15) as float64.

    Written from the bit definition, not from a table: exponent field e,
    mantissa bit m, bias 1; e == 0 is subnormal (0.m * 2**(1-bias)).
    """
    code = np.asarray(code).astype(np.int64)
    sign = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    normal = np.ldexp(1.0 + m / 2.0, (e - E2M1_BIAS).astype(np.int64))
    subnormal = (m / 2.0) * 2.0 ** (1 - E2M1_BIAS)
    mag = np.where(e == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag)


def e2m1_grid():
    """The 8 non-negative E2M1 magnitudes in code order 0..7."""
    return e2m1_decode(np.arange(8))


# Round-to-nearest-even onto the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}:
# a midpoint between two neighbours goes to the neighbour with the even code
# (mantissa bit 0).  Midpoints: 0.25 (->0), 0.75 (->2), 1.25 (->2),
# 1.75 (->4), 2.5 (->4), 3.5 (->6), 5 (->6).  Above 6 saturates to code 7.
def e2m1_encode_magnitude(y):
    """RNE code (0..7) of non-negative magnitudes ``y`` (float32 or float64).

    Counts the midpoints that ``y`` lies above; at a midpoint the comparison
    is strict or not so that the even code wins.
    """
    y = np.asarray(y, dtype=np.float64)
    code = ((y > 0.25).astype(np.int64) + (y >= 0.75) + (y > 1.25) + (y >= 1.75)
            + (y > 2.5) + (y >= 3.5) + (y > 5.0))
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E4M3 ----
# OCP float8_e4m3fn: s|eeee|mmm, bias 7, exponent field 0 is subnormal
# (m/8 * 2**-6), no infinities, 0x7F / 0xFF are NaN, largest finite 448.
E4M3_BIAS = 7
E4M3_MAX = 448.0


def e4m3_decode(byte):
    """float64 value of E4M3 (fn variant) bytes; NaN for 0x7F/0xFF."""
    b = np.asarray(byte).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    sub = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    nor = np.ldexp(1.0 + m / 8.0, (e - E4M3_BIAS).astype(np.int64))
    mag = np.where(e == 0, sub, nor)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode_nonneg(v):
    """E4M3 byte of non-negative values, round-to-nearest-even with
    saturation to 448 (0x7E) above the largest finite value (+inf included).

    Subnormal range (v < 2**-6): the quantum is 2**-9, code = rint(v * 2**9)
    (8 rounds up into the smallest normal, whose byte is also 8).
    Normal range: 2**e <= v < 2**(e+1); m8 = rint(v * 2**(3-e)) in [8, 16];
    16 carries into the next binade.  ``np.rint`` is round-half-even and every
    scaling here is by a power of two, so the arithmetic is exact in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(v < 0):
        raise ValueError("e4m3_encode_nonneg expects non-negative, non-NaN values")
    out = np.full(v.shape, 0x7E, dtype=np.int64)           # saturated default
    sub = v < 2.0 ** (1 - E4M3_BIAS)
    out[sub] = np.rint(v[sub] * 2.0 ** 9).astype(np.int64)
    nor = (~sub) & (v <= E4M3_MAX)
    if np.any(nor):
        vn = v[nor]
        _, ex = np.frexp(vn)            # vn = f * 2**ex, f in [0.5, 1)
        e = ex - 1                      # 2**e <= vn < 2**(e+1)
        m8 = np.rint(np.ldexp(vn, 3 - e)).astype(np.int64)
        carry = m8 == 16
        e = np.where(carry, e + 1, e)
        m8 = np.where(carry, 8, m8)
        out[nor] = ((e + E4M3_BIAS) << 3) | (m8 - 8)
    return out.astype(np.uint8)


# ------------------------------------------------------ bf16 and fp16 ----
def _round_to_precision(x, sig_bits, min_exp, max_finite):
    """Round float64 ``x`` to a binary format with ``sig_bits`` significant
    bits, smallest normal exponent ``min_exp`` (gradual underflow below it)
    and largest finite value ``max_finite``; round-half-even; overflow to inf.
    Exact in float64: the quantum is a power of two and np.rint is RNE."""
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)                 # |x| = f * 2**ex, f in [0.5, 1)
    qexp = np.maximum(ex - sig_bits, min_exp - (sig_bits - 1))
    qexp = np.where(x == 0, 0, qexp)
    r = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
    # Values at or past the midpoint between max_finite and the next (virtual)
    # step overflow; np.rint already produced that next step, so test it.
    r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, x), r)
    return r


BF16_MAX = float.fromhex("0x1.fep127")
FP16_MAX = 65504.0


def bf16_round(x):
    """Round float64/float32 values to the nearest bf16 (RNE); returns float64
    holding bf16 values (8 significant bits, exponent range of fp32)."""
    return _round_to_precision(x, 8, -126, BF16_MAX)


def fp16_round(x):
    """Round to the nearest IEEE binary16 value (RNE, gradual underflow)."""
    return _round_to_precision(x, 11, -14, FP16_MAX)


def bf16_bits(x):
    """uint16 bit pattern of values that are already exactly bf16."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    if np.any((b & 0xFFFF) != 0):
        raise ValueError("values are not exactly representable in bf16")
    return (b >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """float32 values of bf16 bit patterns (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def fp16_bits(x):
    """uint16 bit pattern of values that are already exactly fp16."""
    h = np.asarray(x, dtype=np.float64).astype(np.float16)
    if not np.array_equal(h.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True):
        raise ValueError("values are not exactly representable in fp16")
    return h.view(np.uint16)


def fp16_from_bits(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
