"""GPU parity of int4g_quantize and int4g_gemv against the CPU oracle."""
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


def gpu_int4_quantize(bits):
    q = _q()
    import torch
    N, K = bits.shape
    qq = Guarded((N, K // 2), torch.uint8)
    ss = Guarded((N, K // 128), torch.float16)
    q.int4g_quantize(dev_bf16(bits), out=(qq.t, ss.t))
    torch.cuda.synchronize()
    assert qq.intact() and ss.intact()
    return qq.t, ss.t


def assert_int4_equal(bits, label=""):
    qt, st = gpu_int4_quantize(bits)
    op, osb, _ = I.int4g_quantize(bits)
    gq, gs = host_u8(qt), host_bits(st)
    bad = np.argwhere(gs != osb)
    assert bad.size == 0, f"{label}: {len(bad)} scales differ, first at {bad[0]}"
    bad = np.argwhere(gq != op)
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first at {bad[0]}"
    return qt, st


def test_int4_quantize_worked_group(golden):
    g = golden("int4_worked_example.txt")
    w = np.zeros((1, 128), np.float32)
    w[0, :4] = [float(v) for v in g["w_bf16"]]
    qt, st = assert_int4_equal(F.bf16_bits(w), "worked group")
    assert [int(h, 16) for h in g["bytes_hex"]] == list(host_u8(qt)[0, :2])


@pytest.mark.parametrize("seed,shape,kw", [
    (1, (1, 128), {}), (2, (33, 384), dict(sigma=0.02, outlier_frac=0.005, outlier_mul=10)),
    (3, (64, 1024), dict(zero_frac=0.5)), (4, (5, 256), dict(sigma=1e-6)), (5, (3, 128), dict(sigma=2e4))])
def test_int4_quantize_random(seed, shape, kw):
    assert_int4_equal(workloads.random_bf16(seed, shape, **kw), f"seed {seed}")


def test_int4_quantize_zero_rows():
    z = np.zeros((3, 256), np.uint16)
    assert_int4_equal(z, "zeros")


def gpu_gemv(x_bits, qt, st, algo=0):
    q = _q()
    import torch
    M, N = x_bits.shape[0], qt.shape[0]
    out = Guarded((M, N), torch.bfloat16)
    q.int4g_gemv(dev_bf16(x_bits), qt, st, algo=algo, out=out.t)
    torch.cuda.synchronize()
    assert out.intact()
    return F.bf16_from_bits(host_bits(out.t)).astype(np.float64)


def check_gemv(x_bits, w_bits, algos=(0,), rows=None, label=""):
    qt, st = assert_int4_equal(w_bits, label + " W")
    op, osb, _ = I.int4g_quantize(w_bits)
    xr = x_bits[rows] if rows is not None else x_bits
    ref = I.int4g_gemm(xr, op, osb)
    for algo in algos:
        y = gpu_gemv(x_bits, qt, st, algo)
        ys = y[rows] if rows is not None else y
        ok, rl, rr = Mx.check_output(ys, ref)
        log(f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"
    return qt, st


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 40, 256), (16, 100, 512), (17, 300, 384),
                                   (130, 257, 1024), (256, 512, 256)])
def test_int4_gemv_ragged(M, N, K):
    x = workloads.random_bf16(M + 200, (M, K))
    w = workloads.random_bf16(N + 300, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=10)
    algos = (0, 1, 3) + ((2,) if M <= 16 else ())
    check_gemv(x, w, algos=algos, label=f"int4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 9, 128), (2, 13, 256), (1, 17, 2176), (2, 20, 4096), (1, 3, 32768 + 128),
                                   (3, 65, 384), (7, 130, 2304), (12, 64, 1024), (16, 100, 4224), (9, 47, 128),
                                   (8, 28679, 384), (13, 28800, 256)])
def test_int4_decode_shapes(M, N, K):
    # M <= 2 runs the row-slot GEMV (1 KB slots of 16 groups, partial last
    # slot, ragged N); K > 32768 and 3 <= M <= 16 with K % 512 != 0 run the
    # row-block kernel
    # (64 rows per workgroup, N ragged against it; an odd group count leaves
    # a half step; K = 2304 gives its 8 waves unequal step counts; from M = 8
    # with N >= 112 per compute unit, 112 rows per workgroup, N ragged).
    x = workloads.random_bf16(M + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N + K + 1, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemv(x, w, algos=(0, 2), label=f"int4 decode {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 33, 512), (5, 100, 4608), (16, 16500, 8192), (11, 33769, 1024),
                                   (4, 70, 12288), (16, 1, 512), (8, 129, 4096)])
def test_int4_stationary_shapes(M, N, K):
    # 3 <= M <= 16 with K % 512 == 0 runs the activation-stationary kernel:
    # 512-value pieces per wave and 4096 values per pass (K = 4608 leaves a
    # pass of one piece; K = 12288 takes three passes), 4 or 8 row groups per
    # batch (N >= 64 rows per compute unit takes 8), two batches when a
    # workgroup holds more than 128 rows (N = 33769), N not a multiple of 16.
    x = workloads.random_bf16(M * 7 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 3 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemv(x, w, algos=(0, 2), label=f"int4 stationary {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2, 28672, 8192), (16, 140001, 256), (5, 3000, 12288 + 128), (4, 9, 128),
                                   (2, 300, 65536), (1, 140001, 256), (1, 300, 6144 + 128), (1, 5000, 8192)])
def test_int4_more_decode_shapes(M, N, K):
    # M = 1 on the row-slot GEMV: 17501 workgroups of 8 rows (N = 140001,
    # the last one partial), a partial last slot (K = 6272), four whole
    # slots (K = 8192); the row-slot GEMV at the decode weight's shape with
    # M = 2; the
    # row-block kernel (K % 512 != 0) with 1250 workgroups of 112 rows (N =
    # 140001), an odd group count (K = 12416: a half step at the end) and a
    # lone group (K = 128); K past the row-slot GEMV's limit at M = 2
    x = workloads.random_bf16(M * 11 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w = workloads.random_bf16(N * 13 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemv(x, w, algos=(0, 2), label=f"int4 more {M}x{N}x{K}")


def test_int4_config():
    w = workloads.int4_w()
    x = workloads.int4_x()
    log("int4 config: quantize W [28672, 8192]")
    qt, st = check_gemv(x[:1], w, label="int4 M=1")
    op, osb, _ = I.int4g_quantize(w)
    for M in (2, 16):
        y = gpu_gemv(x[:M], qt, st)
        ok, rl, rr = Mx.check_output(y, I.int4g_gemm(x[:M], op, osb))
        log(f"int4 M={M}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok
    rows = np.random.default_rng(2).choice(2048, 32, replace=False)
    y = gpu_gemv(x, qt, st)
    ok, rl, rr = Mx.check_output(y[rows], I.int4g_gemm(x[rows], op, osb))
    log(f"int4 M=2048 (sampled rows): rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok
