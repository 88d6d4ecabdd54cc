"""The hot path under HIP graph capture.

The library allocates nothing and issues no memsets, so a captured call
sequence replays with fresh inputs: each replay must write the same bits as
the same calls run eagerly on the same inputs, with eager work and
synchronizations between the replays."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import metrics as Mx
from oracle import nvfp4 as O
from tests.gpu_util import dev_bf16, host_bits, log, need_gpu

pytestmark = pytest.mark.gpu


def test_prefill_chain_graph_replays():
    # quantize x -> GEMM up with its amax slots -> quantize h from the slots
    # -> GEMM down; both GEMMs split their last round along K (workspaces).
    torch = need_gpu()
    import quantized_gemm_nvfp4_amd as q
    M, K, N1, N2 = 512, 1024, 2048, 1024
    lib = q.lib()
    w_up_bits = workloads.random_bf16(81, (N1, K), sigma=0.02)
    w_dn_bits = workloads.random_bf16(82, (N2, N1), sigma=0.02)
    w_up = q.nvfp4_quantize(dev_bf16(w_up_bits))
    w_dn = q.nvfp4_quantize(dev_bf16(w_dn_bits))
    dev = "cuda:0"
    x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    a = (torch.empty((M, K // 2), dtype=torch.uint8, device=dev), torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
         torch.empty(1, dtype=torch.float32, device=dev))
    h = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
    hq = (torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev),
          torch.empty((M, N1 // 16), dtype=torch.uint8, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
    y = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
    ws_up = torch.empty(lib.nvfp4_gemm_workspace_bytes(M, N1, K), dtype=torch.uint8, device=dev)
    ws_dn = torch.empty(lib.nvfp4_gemm_workspace_bytes(M, N2, N1), dtype=torch.uint8, device=dev)
    assert ws_up.numel() > 0 and ws_dn.numel() > 0
    slots = torch.empty(lib.nvfp4_gemm_amax_slots(M, N1, K), dtype=torch.int32, device=dev)

    def chain():
        q.nvfp4_quantize(x, out=a)
        q.nvfp4_gemm_amax(a, w_up, out=h, workspace=ws_up, slots=slots)
        q.nvfp4_quantize_amax(h, slots, out=hq)
        q.nvfp4_gemm(hq, w_dn, out=y, workspace=ws_dn)

    x.copy_(dev_bf16(workloads.random_bf16(90, (M, K))))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(4):
        x_bits = workloads.random_bf16(100 + rep, (M, K), outlier_frac=0.01, outlier_mul=10 + rep)
        x.copy_(dev_bf16(x_bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = [host_bits(t) for t in (a[0], a[1], h, hq[0], hq[1], y)]
        chain()
        torch.cuda.synchronize()
        eager = [host_bits(t) for t in (a[0], a[1], h, hq[0], hq[1], y)]
        for name, u, v in zip(("a codes", "a scales", "h", "h codes", "h scales", "y"), replayed, eager):
            assert np.array_equal(u, v), f"replay {rep}: {name} differs from the eager chain"
        if rep == 0:
            # the eager chain itself against the oracle (teacher-forced down
            # projection on the GPU's own h), on sampled rows
            rows = np.sort(np.random.default_rng(4).choice(M, 16, replace=False))
            ref_h = O.gemm_rows(*O.quantize(x_bits), *O.quantize(w_up_bits), rows)
            ok, rl, rr = Mx.check_output(F.bf16_from_bits(eager[2][rows]).astype(np.float64), ref_h)
            assert ok, f"h: rel_l2={rl:.3e} row_ratio={rr:.3e}"
            ref_y = O.gemm_rows(*O.quantize(eager[2]), *O.quantize(w_dn_bits), rows)
            ok, rl, rr = Mx.check_output(F.bf16_from_bits(eager[5][rows]).astype(np.float64), ref_y)
            assert ok, f"y: rel_l2={rl:.3e} row_ratio={rr:.3e}"
        log(f"graph replay {rep}: identical to the eager chain")
