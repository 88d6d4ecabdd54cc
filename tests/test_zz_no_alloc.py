"""GPU test of nvfp4_quantize_noalloc (the entry point that allocates
nothing): through the C ABI, its codes, scales and global scale must equal
nvfp4_quantize's (with a caller workspace) byte for byte, on two calls in a
row, the second on a smaller input, so the second call works on the scratch
the first one left."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev_bf16, log, need_gpu


def _quantize(q, torch, x, noalloc):
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda:0")
    g = torch.empty(1, dtype=torch.float32, device="cuda:0")
    lib = q.lib()
    stream = q._stream(x)
    P = q._ptr
    if noalloc:
        st = lib.nvfp4_quantize_noalloc(P(x), rows, cols, P(codes), P(scales), P(g), 0, stream)
    else:
        ws = torch.empty(lib.nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device="cuda:0")
        st = lib.nvfp4_quantize(P(x), rows, cols, P(codes), P(scales), P(g), 0, P(ws), stream)
    assert st == 0, lib.nvfp4_last_error().decode()
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), g.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    torch = need_gpu()
    import quantized_gemm_nvfp4_amd as q
    # first a two-pass size (more than 2048 blocks, 1024 partial maxima),
    # then a smaller two-pass size (fewer partials: the scratch keeps the
    # first call's values past them) and a single-launch size
    for i, (shape, mul) in enumerate([((512, 5376), 30.0), ((96, 1024), 3.0), ((4, 512), 1.0)]):
        bits = workloads.random_bf16(900 + i, shape, outlier_frac=0.01, outlier_mul=mul, zero_frac=0.02)
        x = dev_bf16(bits)
        log(f"noalloc quantize {shape}")
        want = _quantize(q, torch, x, noalloc=False)
        got = _quantize(q, torch, x, noalloc=True)
        for a, b, name in zip(got, want, ("codes", "scales", "global scale")):
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{shape}: {name} differ"


@pytest.mark.gpu
def test_noalloc_validation_and_given_scale():
    torch = need_gpu()
    import quantized_gemm_nvfp4_amd as q
    lib = q.lib()
    bits = workloads.random_bf16(950, (64, 4096))
    x = dev_bf16(bits)
    codes = torch.empty((64, 2048), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((64, 256), dtype=torch.uint8, device="cuda:0")
    g = torch.full((1,), 0.01, dtype=torch.float32, device="cuda:0")
    P = q._ptr
    assert lib.nvfp4_quantize_noalloc(P(x), 64, 4100, P(codes), P(scales), P(g), 0, q._stream(x)) == 2
    assert lib.nvfp4_quantize_noalloc(P(x), 64, 4096, P(codes), P(codes), P(g), 0, q._stream(x)) == 1
    # given global scale: no first pass, same bytes as nvfp4_quantize with the same g
    assert lib.nvfp4_quantize_noalloc(P(x), 64, 4096, P(codes), P(scales), P(g), 1, q._stream(x)) == 0
    torch.cuda.synchronize()
    c2, s2, _ = q.nvfp4_quantize(x, global_scale=g)
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
