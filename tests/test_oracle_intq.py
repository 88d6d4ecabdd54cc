"""Pins of oracle.intq: the page's worked INT8 example and its outlier
variant, a hand-worked INT4 group, the s/2 error bound, nibble encoding, and
the INT4 GEMM against a pure-Python triple loop."""
import numpy as np

import workloads
from oracle import formats as F
from oracle import intq as I


def _f(lst):
    return np.array([float(v) for v in lst])


def test_page_int8_worked_example(golden):
    g = golden("int8_worked_example.txt")
    s, q, xh = I.symmetric_quantize(_f(g["w"]), int(g["bits"][0]))
    assert abs(s - float(g["s"][0])) <= 1e-5
    assert list(q) == [int(v) for v in g["q"]]
    assert np.all(np.abs(xh - _f(g["x_hat"])) <= 1.0001e-4)
    err = np.abs(_f(g["w"]) - xh)
    assert np.all(np.abs(err - _f(g["abs_err"])) <= 1.0001e-4)
    assert np.all(err <= s / 2 + 1e-15)
    assert abs(s / 2 - float(g["half_s"][0])) <= 1e-4


def test_page_int8_outlier_example(golden):
    g = golden("int8_worked_example.txt")
    w = _f(g["w_out"])
    s, q, xh = I.symmetric_quantize(w, 8)
    assert abs(s - float(g["s_out"][0])) <= 1e-4
    assert list(q[:4]) == [int(v) for v in g["q_out_first4"]]
    assert q[4] == 127
    assert np.all(np.abs(xh[:4] - _f(g["x_hat_out_first4"])) <= 1.0001e-3)
    err = np.abs(w - xh)[:4].max()
    assert err <= float(g["err_out_upper"][0])
    # the outlier makes the small weights' error several times worse
    _, _, xh0 = I.symmetric_quantize(_f(g["w"]), 8)
    assert err / np.abs(_f(g["w"]) - xh0).max() > 8.0


def test_int4_worked_group(golden):
    g = golden("int4_worked_example.txt")
    w = np.zeros((1, 128), np.float32)
    w[0, :4] = _f(g["w_bf16"])
    packed, sbits, q = I.int4g_quantize(w)
    assert F.fp16_from_bits(sbits)[0, 0] == float(g["s16"][0])
    assert list(q[0, :4]) == [int(v) for v in g["q"]]
    assert [int(h, 16) for h in g["bytes_hex"]] == list(packed[0, :2])
    assert not packed[0, 2:].any()


def test_int4_error_bound_and_range():
    for seed, kw in [(1, {}), (2, dict(outlier_frac=0.005, outlier_mul=10)), (3, dict(zero_frac=0.5))]:
        w = F.bf16_from_bits(workloads.random_bf16(seed, (24, 512), sigma=0.02, **kw))
        packed, sbits, q = I.int4g_quantize(w)
        assert q.min() >= -7 and q.max() <= 7
        s = np.repeat(F.fp16_from_bits(sbits), 128, axis=1)
        err = np.abs(w.astype(np.float64) - s * q)
        assert np.all(err <= s / 2 * (1 + 2.0 ** -10) + 1e-300)
        assert np.array_equal(I.int4_unpack(packed), q)
        assert np.array_equal(I.int4g_dequantize(packed, sbits), s * q)


def test_int4_zero_group():
    w = np.zeros((2, 256), np.float32)
    w[1, 130] = 0.5
    packed, sbits, q = I.int4g_quantize(w)
    assert sbits[0, 0] == 0 and sbits[1, 0] == 0 and not q[0].any()
    assert q[1, 130] == 7


def test_int4_nibbles_twos_complement():
    q = np.arange(-7, 8, dtype=np.int8)
    w = np.zeros((1, 128), np.float32)
    w[0, :15] = q.astype(np.float32)          # amax 7 -> s16 = 1
    packed, sbits, qq = I.int4g_quantize(w)
    assert F.fp16_from_bits(sbits)[0, 0] == 1.0
    assert list(qq[0, :15]) == list(q)
    nib = [(int(packed[0, k // 2]) >> (4 * (k % 2))) & 15 for k in range(15)]
    assert nib == [(int(v) + 16) % 16 for v in q]


def test_int4_gemm_vs_triple_loop():
    x = F.bf16_from_bits(workloads.random_bf16(51, (3, 256)))
    w = F.bf16_from_bits(workloads.random_bf16(52, (5, 256), sigma=0.02, outlier_frac=0.01, outlier_mul=10))
    packed, sbits, q = I.int4g_quantize(w)
    s = F.fp16_from_bits(sbits)
    ref = np.zeros((3, 5))
    for i in range(3):
        for j in range(5):
            acc = 0.0
            for k in range(256):
                nib = (int(packed[j, k // 2]) >> (4 * (k % 2))) & 15
                qv = nib - 16 if nib >= 8 else nib
                acc += float(x[i, k]) * float(s[j, k // 128]) * qv
            ref[i, j] = acc
    assert np.allclose(I.int4g_gemm_fp64(x, packed, sbits), ref, rtol=1e-12, atol=1e-15)
    assert np.array_equal(I.int4g_gemm(x, packed, sbits), F.bf16_round(I.int4g_gemm_fp64(x, packed, sbits)))


# ------------------------------------------------------------- asymmetric --
def test_asym_page_formula_worked_group(golden):
    g = golden("int4_asym_worked_example.txt")
    x = np.array([float(t) for t in g["page_values"]])
    s, z, q, xh = I.asymmetric_quantize(x, 4)
    assert s == 5.0 / 15.0 and z == int(g["page_z"][0])
    assert list(q) == [int(t) for t in g["page_q"]]
    assert np.max(np.abs(x - xh)) <= s / 2 + 1e-15


def test_asym_stored_int4_worked_group(golden):
    g = golden("int4_asym_worked_example.txt")
    row = np.zeros((1, 128), dtype=np.float32)
    row[0, :8] = [float(t) for t in g["page_values"]]
    packed, sb, z, q = I.int4g_asym_quantize(F.bf16_bits(row))
    assert sb[0, 0] == int(g["stored_scale_bits"][0], 16)
    assert z[0, 0] == int(g["stored_z"][0])
    assert list(q[0, :8]) == [int(t) for t in g["stored_q8"]]
    assert np.all(q[0, 8:] == 3)
    assert list(packed[0, :4]) == [int(t, 16) for t in g["stored_bytes8"]]
    assert np.all(packed[0, 4:] == 0x33)


def test_asym_bounds_brute_force_and_exact_zero():
    bits = workloads.random_bf16(81, (24, 512), sigma=0.02, outlier_frac=0.01, outlier_mul=10, zero_frac=0.1)
    w = F.bf16_from_bits(bits).astype(np.float64)
    packed, sb, z, q = I.int4g_asym_quantize(bits)
    s = np.repeat(F.fp16_from_bits(sb), 128, axis=1)
    zz = np.repeat(z.astype(np.float64), 128, axis=1)
    xh = I.int4g_asym_dequantize(packed, sb, z)
    err = np.abs(w - xh)
    # zero is exactly representable
    assert np.all(xh[w == 0] == 0)
    # elements whose level was not clamped: within s/2, and at the nearest level
    unclamped = (q > 0) & (q < 15)
    assert np.all(err[unclamped] <= s[unclamped] / 2 * (1 + 1e-6))
    lv = np.arange(16)[None, None, :]
    levels = s[..., None] * (lv - zz[..., None])
    best = np.min(np.abs(w[..., None] - levels), axis=-1)
    assert np.all(err <= best + 1e-12 * np.abs(w).max())
    # everything: within 1.5 s (a clamp at the ends of the widened range)
    assert np.all(err <= 1.5 * s + 1e-12)


def test_asym_zero_group_and_constant_group():
    w = np.zeros((2, 256), dtype=np.float32)
    w[1, 128:] = 0.25                           # one constant positive group
    packed, sb, z, q = I.int4g_asym_quantize(F.bf16_bits(w))
    xh = I.int4g_asym_dequantize(packed, sb, z)
    assert np.all(xh[0] == 0) and np.all(xh[1, :128] == 0)
    np.testing.assert_allclose(xh[1, 128:], 0.25, rtol=2e-3)


def test_asym_gemm_vs_triple_loop():
    rng = np.random.default_rng(9)
    x = F.bf16_round(rng.normal(size=(2, 256)).astype(np.float32)).astype(np.float32)
    w = F.bf16_round((0.02 * rng.normal(size=(3, 256)) + 0.01).astype(np.float32)).astype(np.float32)
    packed, sb, z, q = I.int4g_asym_quantize(F.bf16_bits(w))
    y = I.int4g_asym_gemm_fp64(F.bf16_bits(x), packed, sb, z)
    s = F.fp16_from_bits(sb)
    for m in range(2):
        for n in range(3):
            tot = 0.0
            for k in range(256):
                tot += float(x[m, k]) * float(s[n, k // 128]) * (int(q[n, k]) - int(z[n, k // 128]))
            assert abs(y[m, n] - tot) <= 1e-12 * (1 + abs(tot))
