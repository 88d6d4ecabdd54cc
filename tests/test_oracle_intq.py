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
