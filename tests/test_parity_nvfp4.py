"""GPU parity of nvfp4_quantize and nvfp4_gemm against the CPU oracle.

Codes, scales and the global scale must match byte for byte; GEMM outputs
must satisfy rel-L2 <= 1e-3 and per-row max-abs <= 2e-2 * max|row| against
the oracle's fp64 result rounded to bf16.  Full-size configurations compare
sampled output rows (the oracle evaluates the same definition on those rows
only); codes are compared in full."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import metrics as Mx
from oracle import nvfp4 as O
from tests.gpu_util import Guarded, dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu

ALGOS = {"tiled": 1, "decode": 2, "simple": 3}


def _q():
    need_gpu()
    import quantized_gemm_nvfp4_amd as q
    return q


def gpu_quantize(bits, g=None):
    q = _q()
    import torch
    x = dev_bf16(bits)
    R, C = bits.shape
    codes = Guarded((R, C // 2), torch.uint8)
    scales = Guarded((R, C // 16), torch.uint8)
    gt = torch.tensor([g], dtype=torch.float32, device="cuda:0") if g is not None else None
    out_g = gt if gt is not None else torch.empty(1, dtype=torch.float32, device="cuda:0")
    q.nvfp4_quantize(x, global_scale=gt, out=(codes.t, scales.t, out_g))
    torch.cuda.synchronize()
    assert codes.intact() and scales.intact(), "quantize wrote outside its outputs"
    return codes.t, scales.t, out_g


def assert_quant_equal(bits, g=None, label=""):
    c, s, gg = gpu_quantize(bits, g)
    oc, os_, og = O.quantize(bits, g=g)
    gc, gs, ggv = host_u8(c), host_u8(s), np.float32(gg.cpu().numpy()[0])
    assert ggv.view(np.uint32) == np.float32(og).view(np.uint32), f"{label}: global scale {ggv} != {og}"
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"{label}: {len(bad_s)} scale bytes differ, first at {bad_s[0]}"
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, f"{label}: {len(bad_c)} code bytes differ, first at {bad_c[0]}"
    return c, s, gg


# ------------------------------------------------------------------ quantize
def test_quantize_worked_row(golden):
    g = golden("nvfp4_worked_row.txt")
    vals = np.array([float(v) for v in g["values"]], dtype=np.float32)[None, :]
    bits = F.bf16_bits(vals)
    c, s, gg = assert_quant_equal(bits, label="worked row")
    assert [int(h, 16) for h in g["codes_hex"]] == list(host_u8(c)[0])


@pytest.mark.parametrize("seed,shape,kw", [
    (1, (1, 16), {}),
    (2, (3, 48), {}),
    (3, (37, 272), dict(sigma=0.02, outlier_frac=0.01, outlier_mul=50)),
    (4, (129, 1040), dict(zero_frac=0.2)),
    (5, (64, 4096), dict(sigma=1e-3, outlier_frac=0.001, outlier_mul=1e4)),   # subnormal E4M3 scales
    (6, (7, 160), dict(sigma=1e-36)),                                            # denormal fp32 g
    (7, (2, 2000 * 16), dict(sigma=3e4)),
])
def test_quantize_random(seed, shape, kw):
    log(f"quantize seed={seed} shape={shape}")
    assert_quant_equal(workloads.random_bf16(seed, shape, **kw), label=f"seed {seed}")


@pytest.mark.parametrize("shape", [(8, 4096), (1, 2049 * 16), (4, 5376), (16, 5376), (32, 4096), (1, 8193 * 16),
                                   (3, 1040)])
def test_quantize_single_launch_boundary(shape):
    # up to 8192 blocks one launch takes both passes (one workgroup per 1024
    # blocks, the last one partial, each with its own pass for the maximum);
    # 8193 blocks take the two-pass kernels; both must give the oracle's bytes
    log(f"quantize {shape}")
    assert_quant_equal(workloads.random_bf16(shape[1] + 5, shape, outlier_frac=0.01, outlier_mul=40), label=str(shape))


def test_quantize_degenerate():
    z = np.zeros((4, 64), np.uint16)
    z[1, 3] = 0x8000                                   # -0.0
    assert_quant_equal(z, label="all zero")
    one = np.zeros((3, 32), np.uint16)
    one[2, 31] = F.bf16_bits(np.float32([-2.5]))[0]
    assert_quant_equal(one, label="single value")


def test_quantize_rounding_boundaries():
    # Quotients |x| / d swept in single-ulp steps across every E2M1 rounding
    # boundary (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5): with the given global
    # scale g_j = 2^-7 (1 + j 2^-23), the block maximum 6 * 2^-7 gives scale
    # 1.0, d = g_j, and x = t * 2^-7 lands at t (1 - j 2^-23).  Codes must
    # equal the oracle's (exact fl32 division, ties to even) for every j.
    q = _q()
    import torch
    ts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [6.0 * 2.0 ** -7] + [t * 2.0 ** -7 for t in ts] + [-t * 2.0 ** -7 for t in ts] + [0.0]
    bits = F.bf16_bits(np.array([vals], dtype=np.float32))
    assert np.array_equal(F.bf16_from_bits(bits)[0].astype(np.float64), np.array(vals)), "inputs not bf16-exact"
    g0 = np.float32(2.0 ** -7)
    for j in range(-40, 41):
        gj = g0
        step = np.float32(np.inf) if j > 0 else np.float32(-np.inf)
        for _ in range(abs(j)):
            gj = np.nextafter(gj, step, dtype=np.float32)
        gt = torch.tensor([float(gj)], dtype=torch.float32, device="cuda:0")
        codes, scales, _ = q.nvfp4_quantize(dev_bf16(bits), global_scale=gt)
        torch.cuda.synchronize()
        oc, osc, _ = O.quantize(bits, g=gj)
        assert host_u8(scales)[0, 0] == osc[0, 0] == 0x38, f"j={j}: scale {host_u8(scales)[0, 0]:#x}"
        assert np.array_equal(host_u8(codes), oc), f"j={j}: codes {host_u8(codes)} vs {oc}"


def test_quantize_block_scale_boundaries():
    # The block scale s = (amax / 6) / g (two fp32 divisions, each rounded
    # once) is rounded to E4M3.  With g stepped one ulp at a time around
    # (amax / 6) / t for E4M3 midpoints t (normal, subnormal and next to the
    # largest value), s crosses each midpoint; amax / 6 is exact for amax =
    # 6 and inexact for 7 and 0.625.  Scales and codes must equal the
    # oracle's for every step.
    q = _q()
    import torch
    for amax in (6.0, 7.0, 0.625):
        vals = [amax, -0.5 * amax, 0.375 * amax, -0.75 * amax] + [0.0] * 12
        bits = F.bf16_bits(np.array([vals], dtype=np.float32))
        assert F.bf16_from_bits(bits)[0, 0] == amax
        for t in (1.0625, 1.4375, 17.0, 432.0, 1.5 * 2.0 ** -9, 2.0 ** -7 + 2.0 ** -10):
            g0 = np.float32(np.float32(amax / 6.0) / np.float32(t))
            for j in range(-24, 25):
                gj = g0
                step = np.float32(np.inf) if j > 0 else np.float32(-np.inf)
                for _ in range(abs(j)):
                    gj = np.nextafter(gj, step, dtype=np.float32)
                gt = torch.tensor([float(gj)], dtype=torch.float32, device="cuda:0")
                codes, scales, _ = q.nvfp4_quantize(dev_bf16(bits), global_scale=gt)
                torch.cuda.synchronize()
                oc, osc, _ = O.quantize(bits, g=gj)
                assert host_u8(scales)[0, 0] == osc[0, 0], \
                    f"amax={amax} t={t} j={j}: scale {host_u8(scales)[0, 0]:#x} vs {osc[0, 0]:#x}"
                assert np.array_equal(host_u8(codes), oc), f"amax={amax} t={t} j={j}: codes"


@pytest.mark.parametrize("g", [2.0 ** -60, float(np.nextafter(np.float32(2.0 ** -60), np.float32(0))),
                               2.0 ** 60, float(np.nextafter(np.float32(2.0 ** 60), np.float32(np.inf)))])
def test_quantize_block_scale_range(g):
    # The block-scale step takes reciprocals while g is in [2^-60, 2^60] and
    # the block's amax is 0 or in [2^-60, 2^60], and divides otherwise.  At
    # and just past the bounds of g, blocks whose scale ratio (amax / 6) / g
    # is spread log-uniformly over [2^-12, 2^11] have amax on both sides of
    # the amax bounds; scales and codes must equal the oracle's.
    seed = {2.0 ** -60: 1, 2.0 ** 60: 2}.get(g, 3 if g < 1 else 4)
    bits = workloads.blocks_at_scale_ratio(seed, g, 4096, -12.0, 11.0)
    assert_quant_equal(bits, g=np.float32(g), label=f"g={g!r}")


def test_quantize_given_global_scale():
    bits = workloads.random_bf16(8, (33, 128))
    for g in (1.0, 0.003, 1e-30, 0.0):
        assert_quant_equal(bits, g=g, label=f"given g={g}")


def test_quantize_full_size_tensors():
    x_up, w_up, w_down = workloads.prefill()
    for name, bits in [("prefill x_up", x_up), ("decode/prefill W_up", w_up), ("prefill W_down", w_down),
                       ("decode x", workloads.decode_x()[0]), ("dit x_0", workloads.dit_x(0))]:
        log(f"quantize full {name} {bits.shape}")
        assert_quant_equal(bits, label=name)


def test_quantize_deterministic():
    bits = workloads.random_bf16(9, (300, 512))
    a = gpu_quantize(bits)
    b = gpu_quantize(bits)
    for u, v in zip(a, b):
        assert bool((u == v).all())


# ---------------------------------------------------------------------- gemm
def gpu_gemm(a, w, algo=0):
    q = _q()
    import torch
    M, N = a[0].shape[0], w[0].shape[0]
    out = Guarded((M, N), torch.bfloat16)
    q.nvfp4_gemm(a, w, algo=algo, out=out.t)
    torch.cuda.synchronize()
    assert out.intact(), "gemm wrote outside its output"
    return F.bf16_from_bits(host_bits(out.t)).astype(np.float64)


def check_gemm(a_bits, w_bits, algos=(0,), rows=None, label=""):
    a = assert_quant_equal(a_bits, label=label + " A")
    w = assert_quant_equal(w_bits, label=label + " W")
    oa, ow = O.quantize(a_bits), O.quantize(w_bits)
    ref = O.gemm_rows(*oa, *ow, rows) if rows is not None else O.gemm(*oa, *ow)
    for algo in algos:
        y = gpu_gemm(a, w, algo)
        ys = y[rows] if rows is not None else y
        ok, rl, rr = Mx.check_output(ys, ref)
        log(f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{label} algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}"
    return a, w


def test_gemm_tiny_config_all_kernels():
    a_bits, w_bits = workloads.tiny()
    check_gemm(a_bits, w_bits, algos=(0, 1, 2, 3), label="tiny 16x256x256")


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (5, 37, 256), (16, 300, 384), (17, 33, 128), (100, 250, 640),
    (257, 513, 1024), (300, 260, 128 * 9), (64, 16, 2048)])
def test_gemm_ragged_tiled_and_simple(M, N, K):
    a_bits = workloads.random_bf16(M * 7 + 1, (M, K))
    w_bits = workloads.random_bf16(N * 11 + 2, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=20)
    algos = (0, 1, 3) + ((2,) if M <= 16 else ())
    check_gemm(a_bits, w_bits, algos=algos, label=f"ragged {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,split", [
    (512, 512, 1024, True), (300, 260, 128 * 9, True), (1000, 700, 2048, True), (600, 1300, 256, False)])
def test_gemm_tiled_split_and_whole(M, N, K, split):
    # With a workspace the leftover tiles of the last round are split along
    # K (parts of 4..5 stages, up to 8 parts) and summed by a second kernel;
    # without one every tile runs whole.  Both must meet the bar; the split
    # only changes the fp32 summation order.
    q = _q()
    import torch
    a_bits = workloads.random_bf16(M + 5, (M, K))
    w_bits = workloads.random_bf16(N + 6, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=20)
    a = assert_quant_equal(a_bits, label="split A")
    w = assert_quant_equal(w_bits, label="split W")
    ref = O.gemm(*O.quantize(a_bits), *O.quantize(w_bits))
    nbytes = q.lib().nvfp4_gemm_workspace_bytes(M, N, K)
    assert (nbytes > 0) == split
    outs = {}
    for name, ws in (("split", None), ("whole", torch.empty(0, dtype=torch.uint8, device="cuda:0"))):
        out = Guarded((M, N), torch.bfloat16)
        q.nvfp4_gemm(a, w, algo=q.ALGO_TILED, out=out.t, workspace=ws)
        torch.cuda.synchronize()
        assert out.intact(), "wrote outside its output"
        y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"tiled {name} {M}x{N}x{K}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{name}: rel_l2={rl:.3e} row_ratio={rr:.3e}"
        outs[name] = y
    if not split:
        assert np.array_equal(outs["split"], outs["whole"])


def _random_tiled_shapes(n, seed):
    # Ragged M and N (edge tiles, rows re-read past M or N), K both a
    # multiple of 256 (scale groups and code pairs, loop tails of 4 stages)
    # and an odd multiple of 128 (per-stage copies), grids small enough to
    # be split along K and large enough to run whole rounds.
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        M = int(rng.integers(17, 700))
        N = int(rng.integers(1, 60)) * 16 + (int(rng.integers(0, 16)) if i % 3 else 0)
        K = 128 * (2 * int(rng.integers(1, 13)) + (i % 2))
        shapes.append((M, N, K))
    return shapes


@pytest.mark.parametrize("M,N,K", _random_tiled_shapes(12, 2024))
def test_gemm_tiled_random_shapes(M, N, K):
    # The tiled kernel, with and without a workspace (K split of the last
    # round), against the oracle; with the workspace also its amax variant,
    # whose output bits must equal the plain call's.
    q = _q()
    import torch
    a_bits = workloads.random_bf16(M * 3 + K, (M, K), outlier_frac=0.01, outlier_mul=20)
    w_bits = workloads.random_bf16(N * 5 + K, (N, K), sigma=0.02, zero_frac=0.02)
    a = assert_quant_equal(a_bits, label="random A")
    w = assert_quant_equal(w_bits, label="random W")
    ref = O.gemm(*O.quantize(a_bits), *O.quantize(w_bits))
    outs = []
    for name, ws in (("auto workspace", None), ("no workspace", torch.empty(0, dtype=torch.uint8, device="cuda:0"))):
        out = Guarded((M, N), torch.bfloat16)
        q.nvfp4_gemm(a, w, algo=q.ALGO_TILED, out=out.t, workspace=ws)
        torch.cuda.synchronize()
        assert out.intact(), "wrote outside its output"
        y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)
        ok, rl, rr = Mx.check_output(y, ref)
        log(f"tiled random {M}x{N}x{K} {name}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok, f"{name}: rel_l2={rl:.3e} row_ratio={rr:.3e}"
        outs.append(host_bits(out.t))
    if N % 16 == 0:
        y2, _ = q.nvfp4_gemm_amax(a, w)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y2), outs[0]), "amax variant changed the output"


def test_gemm_tiled_scale_groups_uneven_split():
    # K = 1792 (a multiple of 256): the tiled kernel copies the scale bytes
    # of four stages at once and splits the leftover round (64 of 320 tiles,
    # 4 parts) at whole 4-stage groups, 1 or 2 groups per part; 28 stages is
    # not a multiple of the 8-stage loop.  Checked on sampled rows.
    M, N, K = 4096, 5120, 1792
    q = _q()
    import torch
    a_bits = workloads.random_bf16(71, (M, K))
    w_bits = workloads.random_bf16(72, (N, K), sigma=0.02, outlier_frac=0.005, outlier_mul=20)
    a = assert_quant_equal(a_bits, label="groups A")
    w = assert_quant_equal(w_bits, label="groups W")
    assert q.lib().nvfp4_gemm_workspace_bytes(M, N, K) > 0
    rows = np.sort(np.random.default_rng(3).choice(M, 48, replace=False))
    ref = O.gemm_rows(*O.quantize(a_bits), *O.quantize(w_bits), rows)
    out = Guarded((M, N), torch.bfloat16)
    q.nvfp4_gemm(a, w, algo=q.ALGO_TILED, out=out.t)
    torch.cuda.synchronize()
    assert out.intact(), "wrote outside its output"
    y = F.bf16_from_bits(host_bits(out.t)).astype(np.float64)[rows]
    ok, rl, rr = Mx.check_output(y, ref)
    log(f"tiled scale groups {M}x{N}x{K}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
    assert ok, f"rel_l2={rl:.3e} row_ratio={rr:.3e}"


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (2, 3, 128), (1, 9, 2048), (2, 37, 2176), (1, 33, 4224), (2, 8, 6144), (1, 300, 8192),
    (2, 70, 8192 + 128), (1, 5, 32768 + 128), (1, 140001, 128), (2, 140001, 256)])
def test_gemm_decode_shapes(M, N, K):
    # M <= 2 and K <= 8192 run the streaming GEMV: one 1 KB slot per 2048
    # values of K (the last one partial), rows spread over the grid's waves;
    # with N = 140001 each wave takes more than 64 rows, so its partial sums
    # are flushed from LDS more than once.  8192 < K <= 32768 runs the
    # row-slot GEMV (4 rows per workgroup, N ragged); K > 32768 falls back to
    # the row-block kernel.
    a_bits = workloads.random_bf16(M * 13 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 17 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemm(a_bits, w_bits, algos=(0, 2), label=f"decode {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [
    (3, 17, 128), (4, 40, 2176), (5, 49, 4224), (8, 16, 5376), (9, 50, 2048), (16, 37, 16384),
    (16, 20, 16384 + 128), (12, 64, 6144), (6, 97, 5376), (16, 144, 2304), (11, 95, 33024)])
def test_gemm_rowblock_decode_shapes(M, N, K):
    # 3 <= M <= 16 runs the row-block kernel: 48 W rows per workgroup (N
    # ragged against 48 and against 4), 8 waves taking 256-value steps in
    # turn (K % 256 == 128 leaves a half step; K = 5376 gives the waves
    # unequal step counts; K = 33024 is past the row-slot limit).
    a_bits = workloads.random_bf16(M * 19 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 23 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemm(a_bits, w_bits, algos=(0, 2), label=f"packed decode {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [
    (3, 1, 128), (4, 7, 384), (5, 33, 2176), (8, 1001, 5376), (7, 30001, 256), (4, 61, 8192), (6, 45, 8192 + 128),
    (8, 10, 16384), (3, 257, 16384 + 256)])
def test_gemm_rowblock_ragged_shapes(M, N, K):
    # More row-block shapes: N below one 48-row workgroup and not a multiple
    # of 4, K % 256 == 128 (a half step), K = 8192 and 16384, and N = 30001
    # (626 workgroups, a partial last one).
    a_bits = workloads.random_bf16(M * 29 + K, (M, K), outlier_frac=0.01, outlier_mul=30)
    w_bits = workloads.random_bf16(N * 31 + K, (N, K), sigma=0.02, zero_frac=0.05)
    check_gemm(a_bits, w_bits, algos=(0, 2), label=f"row-block {M}x{N}x{K}")


@pytest.mark.parametrize("K", [16, 48, 80, 272])
def test_gemm_k_not_multiple_of_128_uses_simple(K):
    a_bits = workloads.random_bf16(K + 3, (9, K))
    w_bits = workloads.random_bf16(K + 4, (21, K), sigma=0.02)
    check_gemm(a_bits, w_bits, algos=(0, 3), label=f"K={K}")


def test_gemm_decode_config():
    x_bits, _ = workloads.decode_x()
    w_bits = workloads.decode_w()
    for M in (1, 4, 16):
        check_gemm(x_bits[:M], w_bits, algos=(0,), label=f"decode M={M}")


def test_gemm_prefill_config_chained():
    x_up, w_up, w_down = workloads.prefill()
    rows = np.random.default_rng(0).choice(4096, 48, replace=False)
    rows.sort()
    q = _q()
    a, w = check_gemm(x_up, w_up, algos=(0,), rows=rows, label="prefill up")
    # teacher-forced: the down projection quantizes the GPU's own up output
    h = q.nvfp4_gemm(a, w)
    h_bits = host_bits(h)
    check_gemm(h_bits, w_down, algos=(0,), rows=rows, label="prefill down")


def test_gemm_dit_config_one_step():
    wq, wu, wd = workloads.dit_weights()
    x = workloads.dit_x(0)
    rows = np.random.default_rng(1).choice(4096, 48, replace=False)
    q = _q()
    check_gemm(x, wq, rows=rows, label="dit qkv")
    a, w = check_gemm(x, wu, rows=rows, label="dit up")
    h_bits = host_bits(q.nvfp4_gemm(a, w))
    check_gemm(h_bits, wd, rows=rows, label="dit down")


def test_gemm_deterministic():
    a_bits = workloads.random_bf16(61, (512, 1024))
    w_bits = workloads.random_bf16(62, (768, 1024), sigma=0.02)
    a, w = gpu_quantize(a_bits), gpu_quantize(w_bits)
    for algo in (1, 3):
        y1, y2 = gpu_gemm(a, w, algo), gpu_gemm(a, w, algo)
        assert np.array_equal(y1, y2)
    d1, d2 = gpu_gemm((a[0][:16], a[1][:16], a[2]), w, 2), gpu_gemm((a[0][:16], a[1][:16], a[2]), w, 2)
    assert np.array_equal(d1, d2)


def test_gemm_zero_k_writes_zeros():
    q = _q()
    import torch
    a = (torch.empty((3, 0), dtype=torch.uint8, device="cuda:0"), torch.empty((3, 0), dtype=torch.uint8, device="cuda:0"),
         torch.ones(1, device="cuda:0"))
    w = (torch.empty((5, 0), dtype=torch.uint8, device="cuda:0"), torch.empty((5, 0), dtype=torch.uint8, device="cuda:0"),
         torch.ones(1, device="cuda:0"))
    out = torch.full((3, 5), 7.0, dtype=torch.bfloat16, device="cuda:0")
    q.nvfp4_gemm(a, w, out=out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())


def test_gemm_subnormal_and_zero_scales():
    """Rows spanning 2^-25 in magnitude give subnormal and zero E4M3 block
    scales next to normal ones, in both operands."""
    rng = np.random.default_rng(71)
    a = rng.standard_normal((40, 512)).astype(np.float32)
    a *= (2.0 ** -np.arange(40, dtype=np.float32) * 0.7)[:, None]
    w = rng.standard_normal((72, 512)).astype(np.float32) * 0.02
    w *= (2.0 ** -(np.arange(72, dtype=np.float32) % 25))[:, None]
    w[5, 100] = 3.0
    a_bits = F.bf16_bits(F.bf16_round(a).astype(np.float32))
    w_bits = F.bf16_bits(F.bf16_round(w).astype(np.float32))
    oa, ow = O.quantize(a_bits), O.quantize(w_bits)
    sub = lambda s: np.count_nonzero((s > 0) & (s < 8))
    assert sub(oa[1]) > 0 and sub(ow[1]) > 0, "case must contain subnormal scales"
    check_gemm(a_bits, w_bits, algos=(0, 1, 2, 3) if a_bits.shape[0] <= 16 else (0, 1, 3), label="subnormal scales")
    check_gemm(a_bits[:16], w_bits, algos=(2,), label="subnormal scales decode")
    # M = 1 runs the streaming GEMV: subnormal and zero block scales through
    # its exact 2^-8 scale conversion
    check_gemm(a_bits[:1], w_bits, algos=(0, 2), label="subnormal scales M=1")
    check_gemm(a_bits[20:21], w_bits, algos=(0, 2), label="subnormal scales M=1, small row")
