"""Pins of oracle.nvfp4: the hand-worked row, brute-force scale choice, the
per-element error bound, degenerate blocks, and the GEMM against a
pure-Python triple loop and two special cases."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import nvfp4 as Q


def _bf16_vals(bits):
    return F.bf16_from_bits(bits)


def test_worked_row(golden):
    g = golden("nvfp4_worked_row.txt")
    vals = np.array([float(v) for v in g["values"]], dtype=np.float32)[None, :]
    assert np.signbit(vals[0, 8])           # the -0 survived parsing
    codes, scales, gs = Q.quantize(vals)
    assert gs == np.float32(float(g["global_scale"][0]))
    assert [int(h, 16) for h in g["scales_hex"]] == list(scales[0])
    assert [int(h, 16) for h in g["codes_hex"]] == list(codes[0])


def test_single_level_scheme_with_given_unit_g():
    # g = 1 reproduces a one-level scheme: the scale is E4M3(amax_b / 6).
    x = np.array([[3.0] + [0.0] * 15], dtype=np.float32)
    codes, scales, g = Q.quantize(x, g=1.0)
    assert g == 1.0
    assert scales[0, 0] == 0x30                 # 0.5 = 2^-1 -> exponent field 6
    assert codes[0, 0] & 0xF == 7               # 3 / 0.5 = 6


def _random_cases():
    yield workloads.random_bf16(1, (33, 96))
    yield workloads.random_bf16(2, (17, 160), sigma=0.02, outlier_frac=0.01, outlier_mul=50)
    yield workloads.random_bf16(3, (8, 64), sigma=1e-3, zero_frac=0.3)
    a, w = workloads.tiny()
    yield a
    yield w


def test_scale_is_nearest_e4m3_of_absmax_over_6g():
    vals = F.e4m3_decode(np.arange(0, 0x7F))
    for bits in _random_cases():
        x = _bf16_vals(bits)
        codes, scales, g = Q.quantize(x)
        amax_b = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2).astype(np.float64)
        target = amax_b / 6.0 / np.float64(g)
        s = F.e4m3_decode(scales)
        d = np.abs(target[..., None] - vals)
        best = d.min(axis=-1)
        # the chosen scale is a nearest E4M3 value (the fp32 steps can move
        # the target by a few fp32 ulps, far below half an E4M3 step)
        assert np.all(np.abs(s - target) <= best * (1 + 1e-6) + 1e-30)


def test_block_holding_global_max_gets_scale_448():
    for bits in _random_cases():
        x = _bf16_vals(bits)
        codes, scales, g = Q.quantize(x)
        ab = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2)
        r, b = np.unravel_index(np.argmax(ab), ab.shape)
        assert scales[r, b] == 0x7E
        # g * 2688 equals amax to within one fp32 rounding
        assert abs(np.float64(g) * 2688 - ab.max()) <= ab.max() * 2.0 ** -23


def test_error_bound_per_element():
    for bits in _random_cases():
        x = _bf16_vals(bits).astype(np.float64)
        codes, scales, g = Q.quantize(_bf16_vals(bits))
        xh = Q.dequantize(codes, scales, g)
        d = np.repeat((F.e4m3_decode(scales).astype(np.float32) * g).astype(np.float32).astype(np.float64), 16, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            y = np.where(d > 0, np.abs(x) / d, 0.0)
        mag = np.abs(F.e2m1_decode(Q.unpack_codes(codes)))
        gap = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
        inside = y <= 6.0
        err = np.abs(x - xh)
        # RNE onto the grid; the fp32 quotient adds at most 2^-24 relative
        assert np.all(err[inside] <= d[inside] * (gap[inside] / 2 + 6 * 2.0 ** -23) + 1e-300)
        sat = ~inside
        assert np.all(mag[sat] == 6.0)
        # a normal E4M3 scale is within 1/16 of amax_b/(6g), so |y| <= 6.375:
        # saturated elements then lose at most 0.375 d, and every element at
        # most d (half the widest grid gap, 2)
        normal = np.repeat(F.e4m3_decode(scales) >= 2.0 ** -6, 16, axis=1)
        assert np.all(y[normal] <= 6.375 * (1 + 2.0 ** -20))
        assert np.all(err[normal & sat] <= d[normal & sat] * (0.375 + 1e-6) + 1e-300)
        assert np.all(err[normal] <= d[normal] * (1.0 + 1e-6) + 1e-300)


def test_sign_and_zero_blocks():
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, 16:] = np.float32(1.5)
    x[1, 3] = -0.0
    x[1, 20] = -np.float32(2.0 ** -120)        # tiny negative in a nonzero block
    codes, scales, g = Q.quantize(x)
    assert scales[0, 0] == 0 and scales[1, 0] == 0
    c = Q.unpack_codes(codes)
    assert c[1, 3] == 8 and c[0, 0] == 0
    assert c[1, 20] == 8                       # magnitude underflows to 0, sign kept
    z = np.zeros((3, 48), dtype=np.float32)
    z[2, 5] = -0.0
    codes, scales, g = Q.quantize(z)
    assert g == 0 and not scales.any()
    assert set(np.unique(Q.unpack_codes(codes))) <= {0, 8}
    assert Q.unpack_codes(codes)[2, 5] == 8


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((2, 24), dtype=np.float32))
    with pytest.raises(ValueError):
        Q.quantize(np.full((1, 16), 1.0 + 2 ** -12, dtype=np.float32))


def test_pack_order_low_nibble_first():
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 6.0
    x[0, 1] = 0.5
    codes, scales, g = Q.quantize(x)
    assert codes[0, 0] == 0x17


def _triple_loop(ac, asc, ag, wc, wsc, wg):
    M, N, K = ac.shape[0], wc.shape[0], ac.shape[1] * 2
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def val(packed, scl, r, k):
        byte = int(packed[r, k // 2])
        c = (byte >> 4) if k % 2 else (byte & 15)
        v = grid[c & 7] * (-1.0 if c & 8 else 1.0)
        sb = int(scl[r, k // 16])
        e, m = sb >> 3, sb & 7
        s = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        return v * s

    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                acc += val(ac, asc, i, k) * val(wc, wsc, j, k)
            out[i][j] = float(ag) * float(wg) * acc
    return np.array(out)


def test_gemm_vs_triple_loop():
    a = _bf16_vals(workloads.random_bf16(21, (3, 48)))
    w = _bf16_vals(workloads.random_bf16(22, (5, 48), sigma=0.02, outlier_frac=0.05, outlier_mul=30))
    ac, asc, ag = Q.quantize(a)
    wc, wsc, wg = Q.quantize(w)
    ref = _triple_loop(ac, asc, ag, wc, wsc, wg)
    got = Q.gemm_fp64(ac, asc, ag, wc, wsc, wg)
    assert got.shape == (3, 5)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)
    assert np.array_equal(Q.gemm(ac, asc, ag, wc, wsc, wg), F.bf16_round(ref))
    rows = np.array([2, 0])
    assert np.array_equal(Q.gemm_rows(ac, asc, ag, wc, wsc, wg, rows), Q.gemm(ac, asc, ag, wc, wsc, wg)[rows])


def test_gemm_unit_scales_is_plain_grid_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 4, 6, 64
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    one = np.full((M, K // 16), 0x38, np.uint8)
    onew = np.full((N, K // 16), 0x38, np.uint8)
    got = Q.gemm_fp64(ac, one, 1.0, wc, onew, 1.0)
    # decode by table lookup (independent of e2m1_decode) and integer matmul
    table = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)  # 2*value
    A2 = table[Q.unpack_codes(ac)]
    W2 = table[Q.unpack_codes(wc)]
    assert np.array_equal(got * 4, (A2 @ W2.T).astype(np.float64))


def test_gemm_identity_weight_returns_dequantized_activation():
    a = _bf16_vals(workloads.random_bf16(31, (7, 32)))
    ac, asc, ag = Q.quantize(a)
    K = 32
    wc = np.zeros((K, K // 2), np.uint8)
    for j in range(K):
        wc[j, j // 2] |= (2 << 4) if j % 2 else 2          # code 2 = 1.0 on the diagonal
    wsc = np.full((K, K // 16), 0x38, np.uint8)
    y = Q.gemm(ac, asc, ag, wc, wsc, 1.0)
    assert np.array_equal(y, F.bf16_round(Q.dequantize(ac, asc, ag)))


def test_quantize_accepts_bits_and_values_equally():
    bits = workloads.random_bf16(41, (4, 64))
    r1 = Q.quantize(bits)
    r2 = Q.quantize(F.bf16_from_bits(bits))
    assert all(np.array_equal(u, v) for u, v in zip(r1, r2))


def test_w4a16_vs_triple_loop():
    rng = np.random.default_rng(7)
    x = F.bf16_round(rng.normal(size=(3, 32)).astype(np.float32)).astype(np.float32)
    w = F.bf16_round((0.02 * rng.normal(size=(5, 32))).astype(np.float32)).astype(np.float32)
    wc, ws, wg = Q.quantize(w)
    codes = Q.unpack_codes(wc)
    y = Q.gemm_w4a16_fp64(x, wc, ws, wg)
    for m in range(3):
        for n in range(5):
            tot = 0.0
            for k in range(32):
                wv = float(F.e2m1_decode(codes[n, k])) * float(F.e4m3_decode(ws[n, k // 16]))
                tot += float(x[m, k]) * wv
            assert abs(y[m, n] - float(np.float32(wg)) * tot) <= 1e-12 * (1 + abs(y[m, n]))


def test_w4a16_equals_w4a4_when_x_is_dequantized_nvfp4():
    a_bits = workloads.random_bf16(71, (7, 256), outlier_frac=0.02, outlier_mul=10)
    w_bits = workloads.random_bf16(72, (9, 256), sigma=0.02)
    a = Q.quantize(a_bits, g=1.0)
    w = Q.quantize(w_bits)
    x = Q.dequantize_blockscaled(a[0], a[1]).astype(np.float32)     # bf16-exact values
    assert np.array_equal(F.bf16_round(x), x)
    np.testing.assert_array_equal(Q.gemm_w4a16(x, *w), Q.gemm(*a, *w))
