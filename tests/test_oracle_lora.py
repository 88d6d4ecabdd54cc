"""Pins of the low-rank branch oracle (oracle/lora.py)."""
import numpy as np

import workloads
from oracle import formats as F
from oracle import lora as L
from oracle import nvfp4 as Q


def _bf16(a):
    return F.bf16_bits(F.bf16_round(np.asarray(a, dtype=np.float32)).astype(np.float32))


def test_lora_down_and_up_vs_triple_loop():
    rng = np.random.default_rng(3)
    M, K, N, r = 3, 32, 4, 2
    x = _bf16(rng.normal(size=(M, K)))
    ld = _bf16(0.1 * rng.normal(size=(r, K)))
    lu = _bf16(0.1 * rng.normal(size=(N, r)))
    t = L.lora_down(x, ld)
    xv, ldv, luv = (F.bf16_from_bits(a).astype(np.float64) for a in (x, ld, lu))
    a = Q.quantize(x)
    w = Q.quantize(_bf16(0.02 * rng.normal(size=(N, K))))
    y = L.gemm_lora_fp64(*a, *w, t, lu)
    base = Q.gemm_fp64(*a, *w)
    for m in range(M):
        for j in range(r):
            tot = 0.0
            for k in range(K):
                tot += float(xv[m, k]) * float(ldv[j, k])
            assert abs(t[m, j] - tot) <= 1e-12 * (1 + abs(tot))
        for n in range(N):
            corr = 0.0
            for j in range(r):
                tot = 0.0
                for k in range(K):
                    tot += float(xv[m, k]) * float(ldv[j, k])
                corr += tot * float(luv[n, j])
            assert abs(y[m, n] - (base[m, n] + corr)) <= 1e-12 * (1 + abs(y[m, n]))


def test_associativity_against_merged_correction():
    x = workloads.random_bf16(51, (8, 512))
    ld = workloads.random_bf16(52, (16, 512), sigma=0.05)
    lu = workloads.random_bf16(53, (40, 16), sigma=0.05)
    t = L.lora_down(x, ld)
    lu64 = F.bf16_from_bits(lu).astype(np.float64)
    ld64 = F.bf16_from_bits(ld).astype(np.float64)
    x64 = F.bf16_from_bits(x).astype(np.float64)
    np.testing.assert_allclose(t @ lu64.T, x64 @ (lu64 @ ld64).T, rtol=1e-12, atol=1e-12)


def test_zero_factors_reduce_to_the_plain_gemm():
    x = workloads.random_bf16(54, (5, 256))
    w = workloads.random_bf16(55, (9, 256), sigma=0.02)
    a, wq = Q.quantize(x), Q.quantize(w)
    t = L.lora_down(x, np.zeros((16, 256), np.float32))
    y = L.gemm_lora(*a, *wq, t, np.zeros((9, 16), np.float32))
    np.testing.assert_array_equal(y, Q.gemm(*a, *wq))
