"""Pins of oracle.formats against things other than itself: the closed-form
E2M1 grid, a brute-force nearest-grid search, torch's CPU casts, and an
integer bit-level two-candidate search for bf16 / fp16 rounding."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_grid_closed_form():
    # 1-2-1 bits with largest magnitude 6 -> bias 1 -> this grid, in code order.
    assert list(F.e2m1_grid()) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.e2m1_grid().max() == 6.0
    neg = F.e2m1_decode(np.arange(8, 16))
    assert np.all(np.signbit(neg))
    assert list(-neg) == list(F.e2m1_grid())


def _brute_e2m1(y):
    """Nearest grid value by explicit distances; a tie goes to the even code."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    # clip far-out values (the nearest point stays 6) so fp64 distances to
    # different grid points stay distinct
    y = np.minimum(y, 1e6)
    d = np.abs(y[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates choose the even code; otherwise the single one
    codes = np.arange(8)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 99).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 99).min(axis=1)
    ntied = cand.sum(axis=1)
    return np.where(ntied > 1, even_pick, any_pick)


def test_e2m1_encode_vs_bruteforce_dense():
    # Every fp32 within +-4096 ulps of every grid value and every midpoint,
    # plus whole binades [0.125, 8) sampled every 7th bit pattern, plus
    # values above the top of the grid.
    pts = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 8], np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    near = (bits[:, None] + np.arange(-4096, 4097)[None, :]).ravel()
    near = near[(near >= 0) & (near < 0x7F800000)].astype(np.uint32)
    lo = np.float32(0.125).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    sweep = np.arange(lo, hi, 7, dtype=np.uint32)
    big = np.float32([6.0000005, 100.0, 3.0e38, np.inf])
    ys = np.concatenate([near.view(np.float32), sweep.view(np.float32), big])
    ys = ys[ys >= 0]
    got = F.e2m1_encode_magnitude(ys)
    want = _brute_e2m1(ys.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_decode_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    want = b.to(torch.float32).numpy().astype(np.float64)
    got = F.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert F.e4m3_decode(0x7E) == 448.0
    assert F.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_vs_torch_boundaries_and_binades():
    # all fp32 within +-64 ulps of every E4M3 value and midpoint in [0, 464],
    # every fp32 in three whole binades (a subnormal one, 1..2, 256..464),
    # and a random sample of the rest.
    vals = F.e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [464.0]]).astype(np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    near = (bits[:, None] + np.arange(-64, 65)[None, :]).ravel()
    near = near[near >= 0].astype(np.uint32).view(np.float32)
    def binade(a, b):
        return np.arange(np.float32(a).view(np.uint32), np.float32(b).view(np.uint32), dtype=np.uint32).view(np.float32)
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, np.float32(464).view(np.uint32), 2_000_000, dtype=np.uint32).view(np.float32)
    v = np.concatenate([near, binade(2.0 ** -8, 2.0 ** -7), binade(1.0, 2.0), binade(256.0, 464.0), rnd])
    v = v[(v >= 0) & (v <= 464)]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_nonneg(v)
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates_above_448():
    v = np.array([448.0, 448.0001, 464.0, 479.9, 480.0, 1e6, 3e38, np.inf])
    assert np.all(F.e4m3_encode_nonneg(v) == 0x7E)
    with pytest.raises(ValueError):
        F.e4m3_encode_nonneg(np.array([np.nan]))


def test_e4m3_encode_is_nearest_bruteforce():
    vals = F.e4m3_decode(np.arange(0, 0x7F))
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 0.02, 20000)]).astype(np.float32)
    got = F.e4m3_decode(F.e4m3_encode_nonneg(v))
    d = np.abs(v.astype(np.float64)[:, None] - vals[None, :])
    assert np.all(np.abs(got - v) <= d.min(axis=1) + 0.0)


def _two_candidate_round(x64, keep_bits_f64):
    """Round float64 to a format with the same exponent range as float64
    but fewer mantissa bits by integer manipulation of the float64 bits:
    truncate (toward zero), take the next value up, keep the nearer, ties to
    the even (LSB 0) one.  Normal range only."""
    b = x64.view(np.uint64)
    drop = 52 - keep_bits_f64
    mask = np.uint64((1 << drop) - 1)
    lo = b & ~mask
    hi = lo + np.uint64(1 << drop)
    rem = b & mask
    half = np.uint64(1 << (drop - 1))
    lsb = (lo >> np.uint64(drop)) & np.uint64(1)
    up = (rem > half) | ((rem == half) & (lsb == 1))
    return np.where(up, hi, lo).view(np.float64)


def test_bf16_round_vs_torch_fp32_inputs():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F7FFFFF, 2_000_000, dtype=np.uint32)
    # also exact halfway cases
    hw = (rng.integers(0, 0x7F000000, 100_000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([bits, hw]).view(np.float32)
    x = np.concatenate([x, -x])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = F.bf16_round(x)
    assert np.array_equal(got, want)


def test_bf16_round_fp64_inputs_vs_bit_search():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(1_000_000) * np.exp(rng.uniform(-40, 40, 1_000_000))
    want = _two_candidate_round(np.abs(x), 7) * np.sign(x)
    assert np.array_equal(F.bf16_round(x), want)
    # exact halfway in fp64 between two bf16 values
    assert F.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert F.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert np.isinf(F.bf16_round(np.array([3.5e38]))[0])


def test_fp16_round_vs_torch_and_numpy():
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.uniform(-70000, 70000, 500000), rng.standard_normal(500000) * 1e-5,
                        rng.standard_normal(500000)]).astype(np.float32)
    want_t = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    with np.errstate(over="ignore"):
        want_n = x.astype(np.float16).astype(np.float64)
    got = F.fp16_round(x)
    assert np.array_equal(got, want_t)
    assert np.array_equal(got, want_n)


def test_bits_roundtrip():
    x = np.array([0.0, -0.0, 1.0, -2.5, float.fromhex("0x1.fep127")], dtype=np.float32)
    b = F.bf16_bits(x)
    assert list(b[:2]) == [0x0000, 0x8000]
    assert np.array_equal(F.bf16_from_bits(b), x)
    with pytest.raises(ValueError):
        F.bf16_bits(np.array([1.0 + 2 ** -10], dtype=np.float32))
