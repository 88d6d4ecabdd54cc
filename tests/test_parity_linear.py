"""GPU parity of nvfp4_linear (quantize x, then the block-scaled GEMM).

x's codes, scales and g must equal the oracle's quantization byte for byte,
and the output must be bit-identical to nvfp4_quantize followed by
nvfp4_gemm on the same device (the one-kernel paths, the GEMV at M <= 2 and
the row-block GEMM at 3 <= M <= 16 for small x, repeat the quantizer's
arithmetic in their prologues), and within the GEMM tolerance of the
oracle's fp64 product rounded to bf16."""
import numpy as np
import pytest

import workloads
from oracle import metrics as Mx
from oracle import nvfp4 as O
from tests.gpu_util import Guarded, dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu


def _run(x_bits, w_bits, label):
    need_gpu()
    import torch
    import quantized_gemm_nvfp4_amd as q
    M, K = x_bits.shape
    N = w_bits.shape[0]
    x = dev_bf16(x_bits)
    w = q.nvfp4_quantize(dev_bf16(w_bits))
    out = Guarded((M, N), torch.bfloat16)
    xc = Guarded((M, K // 2), torch.uint8)
    xs = Guarded((M, K // 16), torch.uint8)
    xg = torch.full((1,), -1.0, dtype=torch.float32, device="cuda:0")
    log(f"linear {label}: M={M} N={N} K={K}")
    q.nvfp4_linear(x, w, out=out.t, x_out=(xc.t, xs.t, xg))
    torch.cuda.synchronize()
    assert out.intact() and xc.intact() and xs.intact(), f"{label}: wrote outside an output"

    oc, os_, og = O.quantize(x_bits)
    assert np.float32(xg.cpu().numpy()[0]).view(np.uint32) == np.float32(og).view(np.uint32), f"{label}: g"
    assert np.array_equal(host_u8(xs.t), os_), f"{label}: scale bytes differ"
    assert np.array_equal(host_u8(xc.t), oc), f"{label}: code bytes differ"

    two = q.nvfp4_gemm(q.nvfp4_quantize(x), w)
    torch.cuda.synchronize()
    got = host_bits(out.t)
    assert np.array_equal(got, host_bits(two)), \
        f"{label}: {int((got != host_bits(two)).sum())} outputs differ from quantize + gemm"

    ref = O.gemm(oc, os_, og, *O.quantize(w_bits))
    from oracle import formats as F
    ok, rl, rr = Mx.check_output(F.bf16_from_bits(got).astype(np.float64), ref)
    log(f"linear {label}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok, f"{label}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (2, 3, 128), (1, 300, 2048 + 128), (2, 70, 4224), (1, 257, 6144), (2, 129, 8192),
    (2, 140001, 256)])
def test_linear_one_kernel_shapes(M, N, K):
    # M <= 2, K % 128 == 0, K <= 8192: the GEMV quantizes x itself (one to
    # four 2048-value slots, the last partial; N = 140001 flushes each
    # wave's partial sums more than once)
    x_bits = workloads.random_bf16(M * 41 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 43 + K, (N, K), sigma=0.02, zero_frac=0.05)
    _run(x_bits, w_bits, f"fused {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [
    (3, 50, 2176), (4, 97, 5376), (5, 1, 128), (8, 48, 6144), (9, 200, 5376), (12, 130, 4096), (16, 30, 3072),
    (3, 20000, 256)])
def test_linear_one_kernel_rowblock_shapes(M, N, K):
    # 3 <= M <= 16, K % 128 == 0 and M K / 16 <= 3072: every workgroup of
    # the row-block GEMM quantizes all of x into LDS (one to six blocks per
    # thread; 8 x 6144 and 12 x 4096 and 16 x 3072 fill all six), workgroup 0
    # also stores x's codes; N not a multiple of the 48 rows per workgroup
    x_bits = workloads.random_bf16(M * 59 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 61 + K, (N, K), sigma=0.02, zero_frac=0.05)
    _run(x_bits, w_bits, f"fused row-block {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 33, 8192 + 128), (10, 50, 5376), (16, 64, 5376), (40, 300, 1024),
                                   (2, 21, 48), (4, 30, 1040)])
def test_linear_two_kernel_shapes(M, N, K):
    # K past 8192 at M <= 2, M K / 16 past 3072 at 3 <= M <= 16, M > 16 and
    # K % 128 != 0 quantize first, then multiply
    x_bits = workloads.random_bf16(M * 47 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 53 + K, (N, K), sigma=0.02, zero_frac=0.05)
    _run(x_bits, w_bits, f"two-kernel {M}x{N}x{K}")


def test_linear_degenerate_activations():
    # all-zero x (g = 0: every scale and code 0, output 0), a single
    # nonzero value, and values 2^97 next to bf16 subnormals
    w_bits = workloads.random_bf16(5, (96, 1024), sigma=0.02)
    _run(np.zeros((1, 1024), np.uint16), w_bits, "zero x")
    _run(np.zeros((4, 1024), np.uint16), w_bits, "zero x, M = 4")
    one = np.zeros((2, 1024), np.uint16)
    one[1, 517] = 0xC2F6                        # -123.0
    _run(one, w_bits, "one value")
    wide = workloads.random_bf16(6, (2, 1024))
    wide[0, ::16] = 0x7000                      # 2^97
    wide[1, 3::16] = 0x0001                     # the smallest subnormal
    _run(wide, w_bits, "wide range")
    wide5 = workloads.random_bf16(7, (5, 1024))
    wide5[0, ::16] = 0x7000
    wide5[3, 3::16] = 0x0001
    _run(wide5, w_bits, "wide range, M = 5")


def test_linear_decode_config():
    # the 21504 x 5376 decode weight with the first 1, 2, 4 and 8 rows of
    # the decode activation (one kernel each)
    x_bits, _ = workloads.decode_x()
    w_bits = workloads.decode_w()
    for M in (1, 2, 4, 8):
        _run(x_bits[:M], w_bits, f"decode M={M}")
