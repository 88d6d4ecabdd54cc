"""GPU parity of the low-rank branch on an NVFP4 layer against the CPU oracle.

nvfp4_quantize_lora: codes, scales and the global scale byte-equal to the
oracle's NVFP4 quantization; T = X L_down^T within the fp32 summation bound
K 2^-24 sum_k |x_k l_k| of the fp64 value.  nvfp4_gemm_lora: rel-L2 <= 1e-3
and per-row max-abs <= 2e-2 max|row| versus bf16_RNE of the fp64 layer.
"""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import lora as L
from oracle import metrics as Mx
from oracle import nvfp4 as O
from tests.gpu_util import Guarded, dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu


def _q():
    need_gpu()
    import quantized_gemm_nvfp4_amd as q
    return q


def _dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def gpu_quantize_lora(x_bits, down_bits, given_g=None):
    q = _q()
    import torch
    rows, cols = x_bits.shape
    r = down_bits.shape[0]
    codes = Guarded((rows, cols // 2), torch.uint8)
    scales = Guarded((rows, cols // 16), torch.uint8)
    t = Guarded((rows, r), torch.float32)
    g = _dev_f32([given_g]) if given_g is not None else torch.empty(1, dtype=torch.float32, device="cuda:0")
    q.nvfp4_quantize_lora(dev_bf16(x_bits), dev_bf16(down_bits), global_scale=g if given_g is not None else None,
                          out=(codes.t, scales.t, g, t.t))
    torch.cuda.synchronize()
    assert codes.intact() and scales.intact() and t.intact(), "wrote outside an output"
    return codes.t, scales.t, g, t.t


def check_t(t_gpu, x_bits, down_bits, label):
    ref = L.lora_down(x_bits, down_bits)
    xa = np.abs(F.bf16_from_bits(x_bits).astype(np.float64))
    da = np.abs(F.bf16_from_bits(down_bits).astype(np.float64))
    K = x_bits.shape[1]
    bound = (xa @ da.T) * (K * 2.0 ** -24)
    err = np.abs(t_gpu.astype(np.float64) - ref)
    worst = float(np.max(err - bound)) if err.size else 0.0
    rl = Mx.rel_l2(t_gpu, ref)
    log(f"{label}: T rel_l2={rl:.3e} max(err - bound)={worst:.3e}")
    assert np.all(err <= bound), f"{label}: T outside the fp32 summation bound at {np.argwhere(err > bound)[0]}"
    assert rl <= 1e-6, f"{label}: T rel_l2={rl:.3e}"


def check_codes(codes, scales, g, x_bits, label, given_g=None):
    oc, osc, og = O.quantize(x_bits, g=given_g) if given_g is not None else O.quantize(x_bits)
    assert np.float32(g.cpu().numpy()[0]) == og, f"{label}: global scale differs"
    bad = np.argwhere(host_u8(scales) != osc)
    assert bad.size == 0, f"{label}: {len(bad)} scales differ, first at {bad[0]}"
    bad = np.argwhere(host_u8(codes) != oc)
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first at {bad[0]}"
    return oc, osc, og


@pytest.mark.parametrize("rows,cols,r", [(1, 128, 8), (17, 272, 16), (33, 1024, 24), (100, 3072, 128),
                                         (16 * 1024 + 5, 128, 8), (40, 16, 32), (1, 5376, 32), (3, 2064, 8),
                                         (5, 176, 8), (4096, 1024, 16)])
def test_quantize_lora(rows, cols, r):
    # Covers one K slice and several (small row counts split K across
    # workgroups; the second pass sums the slices), grid-stride over row
    # groups (more than 1024 of them), K % 32 == 16 with the half step in
    # either of a wave's two loads, ranks that leave a 16-block partial.
    x = workloads.random_bf16(rows + cols + r, (rows, cols), outlier_frac=0.002, outlier_mul=20)
    down = workloads.random_bf16(rows * 3 + r, (r, cols), sigma=0.02)
    codes, scales, g, t = gpu_quantize_lora(x, down)
    check_codes(codes, scales, g, x, f"{rows}x{cols} r={r}")
    check_t(t.cpu().numpy(), x, down, f"{rows}x{cols} r={r}")


def test_quantize_lora_given_scale():
    x = workloads.random_bf16(7, (48, 512))
    down = workloads.random_bf16(8, (16, 512), sigma=0.02)
    g = np.float32(1.0 / 1024)
    codes, scales, gt, t = gpu_quantize_lora(x, down, given_g=g)
    check_codes(codes, scales, gt, x, "given g", given_g=g)
    check_t(t.cpu().numpy(), x, down, "given g")


def gpu_gemm_lora(a, w, t, up_bits, algo):
    q = _q()
    import torch
    M, N = a[0].shape[0], w[0].shape[0]
    out = Guarded((M, N), torch.bfloat16)
    q.nvfp4_gemm_lora(a, w, t, dev_bf16(up_bits), algo=algo, out=out.t)
    torch.cuda.synchronize()
    assert out.intact(), "wrote outside its output"
    return F.bf16_from_bits(host_bits(out.t)).astype(np.float64)


@pytest.mark.parametrize("M,N,K,r", [(1, 40, 128, 8), (2, 33, 256, 16), (4, 40, 2176, 16), (5, 70, 512, 32),
                                     (16, 64, 384, 128), (9, 97, 1152, 24),
                                     (130, 257, 1024, 32), (300, 200, 256, 64), (64, 96, 144, 8),
                                     (2048, 4096, 512, 32), (2100, 4100, 768, 24)])
def test_gemm_lora(M, N, K, r):
    # T is a seeded fp32 input with full mantissas, so the epilogue's
    # two-part bf16 split of T is exercised.
    q = _q()
    x = workloads.random_bf16(M * 11 + K, (M, K))
    w = workloads.random_bf16(N * 13 + K, (N, K), sigma=0.02)
    up = workloads.random_bf16(N * 17 + r, (N, r), sigma=0.02)
    t = workloads.random_f32(M * 19 + r, (M, r))
    a_d, w_d = q.nvfp4_quantize(dev_bf16(x)), q.nvfp4_quantize(dev_bf16(w))
    oa, ow = O.quantize(x), O.quantize(w)
    assert np.array_equal(host_u8(a_d[0]), oa[0]) and np.array_equal(host_u8(w_d[0]), ow[0])
    ref = L.gemm_lora(*oa, *ow, t, up)
    algos = [0, 3]
    if K % 128 == 0:
        algos.append(1)
        if M <= 16:
            algos.append(2)
    td = _dev_f32(t)
    for algo in algos:
        y = gpu_gemm_lora(a_d, w_d, td, up, algo)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"lora {M}x{N}x{K} r={r} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


def test_gemm_lora_branch_only():
    # K == 0: the NVFP4 product is empty and the output is the branch alone.
    q = _q()
    import torch
    M, N, r = 3, 24, 16
    t = workloads.random_f32(5, (M, r))
    up = workloads.random_bf16(6, (N, r), sigma=0.02)
    a = (torch.empty((M, 0), dtype=torch.uint8, device="cuda:0"),
         torch.empty((M, 0), dtype=torch.uint8, device="cuda:0"), _dev_f32([1.0]))
    w = (torch.empty((N, 0), dtype=torch.uint8, device="cuda:0"),
         torch.empty((N, 0), dtype=torch.uint8, device="cuda:0"), _dev_f32([1.0]))
    y = gpu_gemm_lora(a, w, _dev_f32(t), up, 0)
    ref = F.bf16_round(t.astype(np.float64) @ F.bf16_from_bits(up).astype(np.float64).T)
    ok, rl, rr = Mx.check_output(y, ref)
    assert ok, f"rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("zero", ["x", "w"])
def test_gemm_lora_zero_global_scale(zero):
    # An all-zero activation or weight has global scale 0, so the product
    # term vanishes and the output is the branch alone.  At 128 tiles the
    # tiled kernel adds the branch to its unscaled accumulators as
    # L_up (T / (g_a g_w))^T, which takes a separate path when g_a g_w = 0.
    q = _q()
    M, N, K, r = 2048, 4096, 512, 16
    x = workloads.random_bf16(41, (M, K))
    w = workloads.random_bf16(42, (N, K), sigma=0.02)
    if zero == "x":
        x = np.zeros_like(x)
    else:
        w = np.zeros_like(w)
    up = workloads.random_bf16(43, (N, r), sigma=0.02)
    t = workloads.random_f32(44, (M, r))
    a_d, w_d = q.nvfp4_quantize(dev_bf16(x)), q.nvfp4_quantize(dev_bf16(w))
    oa, ow = O.quantize(x), O.quantize(w)
    assert np.float32((oa if zero == "x" else ow)[2]) == 0.0
    ref = L.gemm_lora(*oa, *ow, t, up)
    for algo in (0, 1):
        y = gpu_gemm_lora(a_d, w_d, _dev_f32(t), up, algo)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"lora zero {zero} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("case", ["tiny", "huge"])
def test_gemm_lora_extreme_global_scale(case):
    # g_a g_w far from 1: a main weight with amax ~1e-36 has a subnormal
    # global scale (T / (g_a g_w) would overflow fp32, and the output is
    # almost entirely the branch); operands ~1e15 give g_a g_w ~1e24 (the
    # branch is negligible).  The tiled kernel then adds the branch after
    # storing the product.
    q = _q()
    M, N, K, r = 2048, 4096, 512, 16
    sx, sw = (1.0, 1e-36) if case == "tiny" else (1e15, 1e15)
    x = workloads.random_bf16(51, (M, K), sigma=sx)
    w = workloads.random_bf16(52, (N, K), sigma=sw)
    up = workloads.random_bf16(53, (N, r), sigma=0.02)
    t = workloads.random_f32(54, (M, r))
    a_d, w_d = q.nvfp4_quantize(dev_bf16(x)), q.nvfp4_quantize(dev_bf16(w))
    oa, ow = O.quantize(x), O.quantize(w)
    assert np.array_equal(host_u8(w_d[0]), ow[0]) and np.array_equal(host_u8(w_d[1]), ow[1])
    gg = np.float32(oa[2]) * np.float32(ow[2])
    assert 0 < gg < 2.0 ** -100 if case == "tiny" else 2.0 ** 70 < gg < 2.0 ** 100
    ref = L.gemm_lora(*oa, *ow, t, up)
    assert np.all(np.isfinite(ref))
    for algo in (0, 1, 3):
        y = gpu_gemm_lora(a_d, w_d, _dev_f32(t), up, algo)
        assert np.all(np.isfinite(y))
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"lora {case} global scale algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"


def test_linear_lora_dit_qkv():
    # The diffusion qkv projection [4096 x 3072] x [9216 x 3072] with a
    # rank-32 adapter, end to end (quantize with the fused down projection,
    # then the GEMM with the branch), checked on sampled rows.
    q = _q()
    import torch
    x = workloads.dit_x(0)
    w = workloads.dit_weights()[0]
    down, up = workloads.dit_lora(32)
    codes, scales, g, t = gpu_quantize_lora(x, down)
    rows = np.sort(np.random.default_rng(3).choice(x.shape[0], 24, replace=False))
    oc, osc, og = O.quantize(x)
    assert np.float32(g.cpu().numpy()[0]) == og
    assert np.array_equal(host_u8(codes)[rows], oc[rows]) and np.array_equal(host_u8(scales)[rows], osc[rows])
    check_t(t.cpu().numpy()[rows], x[rows], down, "dit qkv T")
    w_d = q.nvfp4_quantize(dev_bf16(w))
    ow = O.quantize(w)
    assert np.array_equal(host_u8(w_d[0]), ow[0]) and np.array_equal(host_u8(w_d[1]), ow[1])
    out = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device="cuda:0")
    q.nvfp4_gemm_lora((codes, scales, g), w_d, t, dev_bf16(up), out=out)
    torch.cuda.synchronize()
    y = F.bf16_from_bits(host_bits(out)).astype(np.float64)[rows]
    ref = L.gemm_lora(oc[rows], osc[rows], og, *ow, L.lora_down(x[rows], down), up)
    ok, rl, rr = Mx.check_output(y, ref)
    log(f"dit qkv + lora r=32 (sampled rows): rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok, f"rel_l2={rl:.3e} row_ratio={rr:.3e}"
    # the branch is not negligible at this size: dropping it breaks parity
    base = F.bf16_round(O.gemm_fp64(oc[rows], osc[rows], og, *ow))
    assert Mx.rel_l2(base, ref) > 1e-2
