"""GPU parity of the weight-only NVFP4 GEMM (bf16 activation x NVFP4 weight)
against the CPU oracle: rel-L2 <= 1e-3 and per-row max-abs <= 2e-2 max|row|
versus the fp64 result rounded to bf16."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import metrics as Mx
from oracle import nvfp4 as O
from tests.gpu_util import Guarded, dev_bf16, host_bits, log, need_gpu

pytestmark = pytest.mark.gpu


def _q():
    need_gpu()
    import quantized_gemm_nvfp4_amd as q
    return q


def check(x_bits, w_bits, algos=(0,), label=""):
    q = _q()
    import torch
    w = q.nvfp4_quantize(dev_bf16(w_bits))
    ow = O.quantize(w_bits)
    ref = O.gemm_w4a16(x_bits, *ow)
    M, N = x_bits.shape[0], w_bits.shape[0]
    for algo in algos:
        out = Guarded((M, N), torch.bfloat16)
        q.nvfp4_gemm_w4a16(dev_bf16(x_bits), w, algo=algo, out=out.t)
        torch.cuda.synchronize()
        assert out.intact(), "wrote outside its output"
        y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"w4a16 {label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 37, 256), (1, 33, 4224), (2, 8, 6144), (1, 9, 32768),
                                   (3, 37, 256), (5, 20, 2176), (16, 41, 1024), (1, 140001, 256),
                                   (1, 300, 6144 + 128), (1, 5000, 8192), (2, 140001, 256), (2, 300, 6144 + 128)])
def test_decode_shapes(M, N, K):
    # M = 1 with K <= 8192 runs the streaming GEMV (N = 140001: each wave
    # takes more than 64 rows; K = 6272: a partial last slot), larger K the
    # row-slot GEMV; M = 2 the row band, past its K the row-slot GEMV
    x = workloads.random_bf16(M * 3 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 5 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check(x, w, algos=(0, 2, 3), label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4, 300, 6272), (7, 20000, 8192), (16, 70, 12288), (9, 33000, 6656),
                                   (3, 1, 6272), (12, 17, 8704)])
def test_stationary_shapes(M, N, K):
    # 3 <= M <= 16 with K > 6144 runs the activation-stationary kernel:
    # 512-value pieces per wave, 7 waves x 2 passes for K = 6272 (a quarter
    # piece at the end of each row), 8 x 2 for 8192, 8 x 3 for 12288, 8 row
    # groups per batch when N >= 64 rows per compute unit (N = 20000) and two
    # batches when a workgroup holds more than 128 rows (N = 33000), N not a
    # multiple of 16.
    x = workloads.random_bf16(M * 13 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 17 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check(x, w, algos=(0, 2), label=f"stationary {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4, 300, 5376), (7, 20000, 4096), (9, 33000, 512), (3, 1, 128), (12, 17, 4608),
                                   (16, 4100, 2176), (5, 140001, 256), (8, 21504, 6144), (16, 31, 6016),
                                   (2, 20000, 5376), (2, 45, 128)])
def test_band_shapes(M, N, K):
    # 2 <= M <= 16 with K <= 6144 runs the row-band kernel: one workgroup per
    # CU over contiguous bands of 16-row groups (N = 4100: one or two groups
    # per workgroup; N = 140001: more than eight, so several passes through
    # the band), waves owning 1-3 steps of 256 values (K = 128 and 512 leave
    # waves without steps; K = 2176 and 6016 end with a half step; K = 6144
    # gives every wave three), N not a multiple of 16.
    x = workloads.random_bf16(M * 19 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 23 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check(x, w, algos=(0, 2), label=f"band {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(17, 40, 272), (1, 5, 32768 + 128), (5, 3, 16)])
def test_simple_shapes(M, N, K):
    x = workloads.random_bf16(M * 7 + K, (M, K))
    w = workloads.random_bf16(N * 11 + K, (N, K), sigma=0.02)
    check(x, w, algos=(0, 3), label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("scale", [1e-30, 1e-6, 1e20])
@pytest.mark.parametrize("M", [1, 2, 5])
def test_activation_range_rescaling(scale, M):
    # the decode kernels rescale x by a power of two per 2048-value slot (M
    # <= 2) or per row and wave slice (M >= 3: 512-value pieces, or a wave's
    # steps in the row-band kernel) before the fp16 conversion: tiny and huge
    # activations stay within tolerance
    x = (workloads.random_bf16(91, (M, 2048 * 3)).view(np.uint16))
    xv = (F.bf16_from_bits(x).astype(np.float64) * scale).astype(np.float32)
    xb = F.bf16_bits(F.bf16_round(xv).astype(np.float32))
    w = workloads.random_bf16(92, (24, 2048 * 3), sigma=0.02)
    check(xb, w, algos=(2,), label=f"x*{scale:g}")


@pytest.mark.parametrize("M", [1, 4])
def test_wide_dynamic_range_within_a_slot(M):
    rng = np.random.default_rng(93)
    K = 4096
    mag = np.ldexp(1.0, rng.integers(-24, 12, size=(M, K))) * rng.choice([-1, 1], size=(M, K))
    xb = F.bf16_bits(F.bf16_round(mag.astype(np.float32)).astype(np.float32))
    w = workloads.random_bf16(94, (40, K), sigma=0.02)
    check(xb, w, algos=(2,), label=f"2^-24..2^12 M={M}")


def test_decode_config():
    x_bits, _ = workloads.decode_x()
    w_bits = workloads.decode_w()
    for M in (1, 2, 3, 4, 16):
        check(x_bits[:M], w_bits, algos=(0,), label=f"decode M={M}")


@pytest.mark.parametrize("M,N,K", [(17, 37, 128), (64, 256, 1024), (130, 300, 2176), (300, 513, 384),
                                   (33, 20, 6272), (2048, 512, 5376)])
def test_tiled_shapes(M, N, K):
    # M > 16 with K % 128 == 0 runs the LDS-staged MFMA tiles (128 x 256,
    # one 128-value stage per step): partial tiles along M and N, one to 49
    # stages (the unrolled stage loop and its checked tail), several rows of
    # tiles at M = 2048.  bf16 x goes to the matrix cores as it is, so the
    # products are exact whatever its range.
    x = workloads.random_bf16(M * 19 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 23 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check(x, w, algos=(0, 1, 3), label=f"tiled {M}x{N}x{K}")


def test_tiled_wide_range():
    # activations 2^60 and 2^-60 apart in one row, all-zero weight rows and
    # a weight row of one repeated block: the tiled path needs no rescaling
    M, N, K = 40, 96, 512
    x = workloads.random_bf16(7, (M, K))
    x[0, ::7] = 0x5D80          # 2^60 (sign clear)
    x[1, 3::5] = 0x2180         # 2^-60
    w = workloads.random_bf16(8, (N, K), sigma=0.02)
    w[5] = 0
    w[6] = np.tile(w[7, :16], K // 16)
    check(x, w, algos=(1, 3), label="tiled wide range")


def test_tiled_prefill_shape_sampled():
    # The weight-only call bench.py times past decode sizes: the prefill
    # activation [4096 x 5376] times the 21504 x 5376 decode weight, through
    # the MFMA tiles; 32 sampled rows against the oracle (x is not quantized,
    # so a row of the output depends only on that row of x).
    q = _q()
    import torch
    x_bits = workloads.normal_bf16("prefill", 0, (4096, 5376))
    w_bits = workloads.decode_w()
    w = q.nvfp4_quantize(dev_bf16(w_bits))
    out = Guarded((4096, 21504), torch.bfloat16)
    q.nvfp4_gemm_w4a16(dev_bf16(x_bits), w, out=out.t)
    torch.cuda.synchronize()
    assert out.intact(), "wrote outside its output"
    rows = np.sort(np.random.default_rng(11).choice(4096, 32, replace=False))
    ref = O.gemm_w4a16(x_bits[rows], *O.quantize(w_bits))
    y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)[rows]
    ok, rl, rr = Mx.check_output(y, ref)
    log(f"w4a16 tiled prefill shape (sampled): rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok, f"rel_l2={rl:.3e} row_ratio={rr:.3e}"
