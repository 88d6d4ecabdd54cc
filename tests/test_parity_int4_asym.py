"""GPU parity of the asymmetric (zero-point) INT4 per-group path against the
CPU oracle: codes, fp16 scales and zero points byte-equal; GEMV outputs within
rel-L2 <= 1e-3 and per-row max-abs <= 2e-2 max|row|."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import intq as I
from oracle import metrics as Mx
from tests.gpu_util import Guarded, dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu


def _q():
    need_gpu()
    import quantized_gemm_nvfp4_amd as q
    return q


def gpu_quantize(bits):
    q = _q()
    import torch
    N, K = bits.shape
    qq = Guarded((N, K // 2), torch.uint8)
    ss = Guarded((N, K // 128), torch.float16)
    zz = Guarded((N, K // 128), torch.uint8)
    q.int4g_asym_quantize(dev_bf16(bits), out=(qq.t, ss.t, zz.t))
    torch.cuda.synchronize()
    assert qq.intact() and ss.intact() and zz.intact()
    return qq.t, ss.t, zz.t


def assert_equal(bits, label="", rows=None):
    qt, st, zt = gpu_quantize(bits)
    sub = bits if rows is None else bits[rows]
    op, osb, oz, _ = I.int4g_asym_quantize(sub)
    gq, gs, gz = host_u8(qt), host_bits(st), host_u8(zt)
    if rows is not None:
        gq, gs, gz = gq[rows], gs[rows], gz[rows]
    for name, a, b in (("scales", gs, osb), ("zeros", gz, oz), ("codes", gq, op)):
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{label}: {len(bad)} {name} differ, first at {bad[0]}"
    return qt, st, zt


def test_worked_group(golden):
    g = golden("int4_asym_worked_example.txt")
    row = np.zeros((1, 128), dtype=np.float32)
    row[0, :8] = [float(t) for t in g["page_values"]]
    qt, st, zt = assert_equal(F.bf16_bits(row), "worked group")
    assert list(host_u8(qt)[0, :4]) == [int(t, 16) for t in g["stored_bytes8"]]


@pytest.mark.parametrize("seed,shape,kw", [
    (1, (1, 128), {}), (2, (33, 384), dict(sigma=0.02, outlier_frac=0.005, outlier_mul=10)),
    (3, (64, 1024), dict(zero_frac=0.5)), (4, (5, 256), dict(sigma=1e-6)), (5, (3, 128), dict(sigma=2e4))])
def test_quantize_random(seed, shape, kw):
    assert_equal(workloads.random_bf16(300 + seed, shape, **kw), f"random {shape}")


def test_quantize_one_signed_and_constant_groups():
    w = F.bf16_from_bits(workloads.random_bf16(311, (6, 512), sigma=0.05)).astype(np.float32)
    w[0] = np.abs(w[0])            # all positive: lo = 0
    w[1] = -np.abs(w[1])           # all negative: hi = 0
    w[2, :128] = 0.375             # constant groups
    w[2, 128:256] = -3.0
    w[3, :256] = 0.0               # zero groups
    assert_equal(F.bf16_bits(F.bf16_round(w).astype(np.float32)), "signed/constant groups")


def check_gemv(x_bits, w_bits, algos=(0,), label=""):
    q = _q()
    import torch
    qt, st, zt = assert_equal(w_bits, label + " W")
    op, osb, oz, _ = I.int4g_asym_quantize(w_bits)
    ref = I.int4g_asym_gemm(x_bits, op, osb, oz)
    M, N = x_bits.shape[0], w_bits.shape[0]
    for algo in algos:
        out = Guarded((M, N), torch.bfloat16)
        q.int4g_asym_gemv(dev_bf16(x_bits), qt, st, zt, algo=algo, out=out.t)
        torch.cuda.synchronize()
        assert out.intact()
        y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"int4 asym {label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("M,N,K", [(1, 9, 128), (2, 13, 256), (1, 17, 2176), (2, 20, 4096), (1, 3, 32768 + 128),
                                   (3, 40, 256), (17, 30, 384)])
def test_gemv_shapes(M, N, K):
    x = workloads.random_bf16(M + K + 7, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N + K + 8, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=10)
    algos = (0, 1, 3) + ((2,) if M <= 2 and K <= 32768 else ())
    check_gemv(x, w, algos=algos, label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 40, 256), (130, 257, 1024), (256, 512, 256), (16, 300, 8192),
                                   (64, 1000, 4224), (200, 37, 128)])
def test_tiled_shapes(M, N, K):
    # M >= 3 runs the tile kernel: 128 x 256 tiles, ragged in both (M = 130,
    # 200; N = 257, 300, 37), one group (K = 128), an odd group count (4224)
    x = workloads.random_bf16(M * 5 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 7 + K, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=10)
    check_gemv(x, w, algos=(0, 1), label=f"tiled {M}x{N}x{K}")


def test_config_sampled():
    q = _q()
    import torch
    w = workloads.int4_w()
    x = workloads.int4_x()
    rows = np.sort(np.random.default_rng(12).choice(w.shape[0], 64, replace=False))
    log("int4 asym config: quantize W [28672, 8192] on the GPU, oracle on 64 rows")
    qt, st, zt = assert_equal(w, "config W", rows=rows)
    op, osb, oz, _ = I.int4g_asym_quantize(w[rows])
    for M in (1, 2, 16):
        y = q.int4g_asym_gemv(dev_bf16(x[:M]), qt, st, zt)
        torch.cuda.synchronize()
        yv = F.bf16_from_bits(host_bits(y)).astype(np.float64)[:, rows]
        ok, rl, rr = Mx.check_output(yv, I.int4g_asym_gemm(x[:M], op, osb, oz))
        log(f"int4 asym M={M} (64 sampled columns): rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok
    # M = 2048 on the tile kernel: 16 sampled rows of x against the 64 columns
    xr = np.sort(np.random.default_rng(13).choice(2048, 16, replace=False))
    y = q.int4g_asym_gemv(dev_bf16(x), qt, st, zt)
    torch.cuda.synchronize()
    yv = F.bf16_from_bits(host_bits(y)).astype(np.float64)[xr][:, rows]
    ok, rl, rr = Mx.check_output(yv, I.int4g_asym_gemm(x[xr], op, osb, oz))
    log(f"int4 asym M=2048 (16 x 64 sampled): rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok
