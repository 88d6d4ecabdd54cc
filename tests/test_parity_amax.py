"""GPU parity of the fused-amax pair nvfp4_gemm_amax / nvfp4_quantize_amax.

nvfp4_gemm_amax must write the same output bits as nvfp4_gemm (same
workspace, so the same kernel and summation order), overwrite every amax
slot with a bf16 magnitude pattern whose largest value is max|out|, and in
the tiled kernel one slot per 256 x 256 output tile holding that tile's
maximum.  Quantizing the output from the slots must reproduce the oracle's
codes, scales and global scale for that output byte for byte (and thus
nvfp4_quantize's)."""
import numpy as np
import pytest

import workloads
from oracle import nvfp4 as O
from tests.gpu_util import dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FFFFFFF      # not a bf16 magnitude pattern: a slot left unwritten shows


def _tile_maxima(mag, tm=256, tn=256):
    M, N = mag.shape
    return sorted(int(mag[i:i + tm, j:j + tn].max()) for i in range(0, M, tm) for j in range(0, N, tn))


@pytest.mark.parametrize("M,N,K,split", [
    (512, 4096, 2048, True),     # 32 tiles; the partial last round is split 8 ways along K
    (512, 4096, 2048, False),    # same shape, every tile whole
    (300, 272, 1152, True),      # ragged edge tiles, split 4 ways
    (8, 160, 256, False),        # decode kernel, then a separate pass over the output
    (40, 48, 144, False),        # simple kernel (K % 128 != 0), then a separate pass
])
def test_gemm_amax(M, N, K, split):
    torch = need_gpu()
    import quantized_gemm_nvfp4_amd as q
    log(f"gemm_amax {M}x{N}x{K} split={split}")
    a = q.nvfp4_quantize(dev_bf16(workloads.random_bf16(M + K, (M, K), outlier_frac=0.01, outlier_mul=30)))
    w = q.nvfp4_quantize(dev_bf16(workloads.random_bf16(N + K + 7, (N, K), sigma=0.02, zero_frac=0.05)))
    nbytes = q.lib().nvfp4_gemm_workspace_bytes(M, N, K)
    if split:
        assert nbytes > 0
    ws = torch.empty(nbytes if split else 0, dtype=torch.uint8, device="cuda:0")
    nslots = q.lib().nvfp4_gemm_amax_slots(M, N, K)
    tiled = M > 16 and K % 128 == 0
    if tiled:
        assert nslots == ((M + 255) // 256) * ((N + 255) // 256)
    slots = torch.full((nslots + 3,), SENTINEL, dtype=torch.int32, device="cuda:0")
    out, used = q.nvfp4_gemm_amax(a, w, workspace=ws, slots=slots)
    ref = q.nvfp4_gemm(a, w, workspace=ws)
    torch.cuda.synchronize()
    assert used.numel() == nslots
    ob = host_bits(out)
    assert np.array_equal(ob, host_bits(ref)), "output differs from nvfp4_gemm"
    sl = used.cpu().numpy().astype(np.int64)
    assert (sl <= 0x7FFF).all(), "an amax slot was not written"
    assert (slots[nslots:].cpu().numpy() == SENTINEL).all(), "wrote past the slots"
    mag = (ob & 0x7FFF).astype(np.int64)
    assert sl.max() == mag.max()
    if tiled:
        assert sorted(sl.tolist()) == _tile_maxima(mag), "slots are not the per-tile maxima"
    c, s, g = q.nvfp4_quantize_amax(out, used)
    oc, os_, og = O.quantize(ob)
    assert np.float32(g.cpu().numpy()[0]).view(np.uint32) == np.float32(og).view(np.uint32)
    assert np.array_equal(host_u8(s), os_), "scales differ from the oracle"
    assert np.array_equal(host_u8(c), oc), "codes differ from the oracle"


def test_quantize_amax_matches_quantize():
    # slots produced some other way (here: the per-row maxima) give the same
    # result as the quantizer's own pass, whatever their number
    torch = need_gpu()
    import quantized_gemm_nvfp4_amd as q
    bits = workloads.random_bf16(11, (37, 272), sigma=0.02, outlier_frac=0.01, outlier_mul=50)
    x = dev_bf16(bits)
    rows = (bits & 0x7FFF).astype(np.int64).max(axis=1).astype(np.int32)
    slots = torch.from_numpy(rows).to("cuda:0")
    c, s, g = q.nvfp4_quantize_amax(x, slots)
    c2, s2, g2 = q.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2)
