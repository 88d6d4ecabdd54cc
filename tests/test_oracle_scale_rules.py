"""Pins of the block-scale selection rules (absmax, four-over-six, MSE)."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import nvfp4 as O
from oracle import scale_rules as S


def _row(values):
    v = np.array([float(t) for t in values], dtype=np.float32)[None, :]
    return F.bf16_bits(v)


def _hex(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint8)


def test_hand_worked_block_a(golden):
    g = golden("nvfp4_scale_rules_block.txt")
    bits = _row(g["a_values"])
    for rule in ("absmax", "four_over_six", "mse"):
        codes, scales, _ = S.quantize(bits, rule=rule, g=1.0)
        assert scales[0, 0] == int(g[f"a_{rule}_scale"][0], 16), rule
        assert np.array_equal(codes[0], _hex(g[f"a_{rule}_bytes"])), rule
    codes, scales, _ = S.quantize(bits, rule="absmax", g=1.0)
    err = S.reconstruction_error(bits, codes, scales, 1.0)
    assert err[0, 0] == np.float32(float(g["a_absmax_error"][0]))


def test_hand_worked_block_b_no_rule_improves_an_exact_block(golden):
    g = golden("nvfp4_scale_rules_block.txt")
    bits = _row(g["b_values"])
    for rule in S.RULES:
        codes, scales, _ = S.quantize(bits, rule=rule, g=1.0)
        assert scales[0, 0] == int(g["b_scale"][0], 16), rule
        assert np.array_equal(codes[0], _hex(g["b_bytes"])), rule


def test_absmax_rule_is_the_plain_quantizer():
    bits = workloads.random_bf16(21, (40, 512), outlier_frac=0.01, outlier_mul=30, zero_frac=0.1)
    a = O.quantize(bits)
    b = S.quantize(bits, rule="absmax")
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u), np.asarray(v))


def test_error_ordering_absmax_ge_four_over_six_ge_mse():
    bits = workloads.random_bf16(22, (64, 1024), sigma=0.02, outlier_frac=0.02, outlier_mul=20)
    errs = {}
    for rule in S.RULES:
        c, s, g = S.quantize(bits, rule=rule)
        errs[rule] = S.reconstruction_error(bits, c, s, g)
    assert np.all(errs["four_over_six"] <= errs["absmax"])
    assert np.all(errs["mse"] <= errs["four_over_six"])
    # the rules change something on random data, and reduce the total error
    assert errs["mse"].sum() < errs["four_over_six"].sum() < errs["absmax"].sum()


def _exact_block_on_scale(s_code, pattern):
    """16 bf16 values grid[pattern] * E4M3(s_code) (all exact in bf16)."""
    grid = F.e2m1_grid()
    s = F.e4m3_decode(np.uint8(s_code))
    return (grid[np.asarray(pattern)] * s).astype(np.float32)


@pytest.mark.parametrize("s_code,pattern", [
    (0x34, [6, 5, 5, 5, 2, 2, 2, 2, 1, 1, 0, 0, 3, 3, 4, 4]),   # max 4 s*: four-over-six finds it
    (0x3C, [6, 6, 6, 6, 1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3]),   # max 4 s*
    (0x2A, [5, 3, 3, 1, 0, 0, 1, 2, 5, 4, 4, 3, 2, 1, 1, 1]),   # max 3 s*: absmax scale s*/2 also exact
])
def test_blocks_exact_under_an_in_window_scale_get_zero_error(s_code, pattern):
    vals = _exact_block_on_scale(s_code, pattern)[None, :]
    bits = F.bf16_bits(vals)
    for rule in ("four_over_six", "mse"):
        c, s, g = S.quantize(bits, rule=rule, g=1.0)
        err = S.reconstruction_error(bits, c, s, g)
        assert err[0, 0] == 0.0, (rule, hex(s[0, 0]))
        np.testing.assert_array_equal(O.dequantize(c, s, g)[0], vals[0].astype(np.float64))


def test_mse_choice_is_the_window_minimum_by_brute_force():
    """Independent search: for each block, evaluate every in-window E4M3
    scale with float64 arithmetic (plain Python loops) and check that the
    oracle's choice attains the minimum up to fp32 rounding of the error."""
    bits = workloads.random_bf16(23, (6, 256), outlier_frac=0.05, outlier_mul=15)
    xf = F.bf16_from_bits(bits).astype(np.float64)
    c, s, g = S.quantize(bits, rule="mse")
    g64 = float(np.float32(g))
    grid = list(F.e2m1_grid())
    for r in range(xf.shape[0]):
        for b in range(xf.shape[1] // 16):
            blk = xf[r, 16 * b:16 * b + 16]
            amax = max(abs(t) for t in blk)
            c6 = int(F.e4m3_encode_nonneg(np.float32(np.float32(np.float32(amax) / np.float32(6)) / np.float32(g))))

            def err64(code):
                d = float(F.e4m3_decode(np.uint8(code))) * g64
                tot = 0.0
                for t in blk:
                    y = abs(t) / d if d else 0.0
                    # nearest grid value, ties to the even index
                    best = min(range(8), key=lambda i: (abs(grid[i] - y), i % 2))
                    v = grid[best] * (1 if t >= 0 else -1)
                    tot += (t - v * d) ** 2
                return tot
            cands = [k for k in range(c6 - 8, c6 + 9) if 1 <= k <= 0x7E] or [c6]
            emin = min(err64(k) for k in cands)
            echo = err64(int(s[r, b]))
            assert echo <= emin * (1 + 1e-5) + 1e-30, (r, b, hex(int(s[r, b])), echo, emin)
