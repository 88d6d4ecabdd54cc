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
                                   (3, 37, 256), (5, 20, 2176), (16, 41, 1024)])
def test_decode_shapes(M, N, K):
    x = workloads.random_bf16(M * 3 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 5 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check(x, w, algos=(0, 2, 3), label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(17, 40, 272), (1, 5, 32768 + 128), (5, 3, 16)])
def test_simple_shapes(M, N, K):
    x = workloads.random_bf16(M * 7 + K, (M, K))
    w = workloads.random_bf16(N * 11 + K, (N, K), sigma=0.02)
    check(x, w, algos=(0, 3), label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("scale", [1e-30, 1e-6, 1e20])
def test_activation_range_rescaling(scale):
    # the decode kernel rescales each slot of x by a power of two before the
    # fp16 conversion: tiny and huge activations stay within tolerance
    x = (workloads.random_bf16(91, (2, 2048 * 3)).view(np.uint16))
    xv = (F.bf16_from_bits(x).astype(np.float64) * scale).astype(np.float32)
    xb = F.bf16_bits(F.bf16_round(xv).astype(np.float32))
    w = workloads.random_bf16(92, (24, 2048 * 3), sigma=0.02)
    check(xb, w, algos=(2,), label=f"x*{scale:g}")


def test_wide_dynamic_range_within_a_slot():
    rng = np.random.default_rng(93)
    K = 4096
    mag = np.ldexp(1.0, rng.integers(-24, 12, size=(1, K))) * rng.choice([-1, 1], size=(1, K))
    xb = F.bf16_bits(F.bf16_round(mag.astype(np.float32)).astype(np.float32))
    w = workloads.random_bf16(94, (40, K), sigma=0.02)
    check(xb, w, algos=(2,), label="2^-24..2^12")


def test_decode_config():
    x_bits, _ = workloads.decode_x()
    w_bits = workloads.decode_w()
    for M in (1, 2, 3, 16):
        check(x_bits[:M], w_bits, algos=(0,), label=f"decode M={M}")
