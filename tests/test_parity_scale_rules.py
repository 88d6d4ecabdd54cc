"""GPU parity of nvfp4_quantize_ex's block-scale rules (absmax, four-over-six,
MSE) against the CPU oracle: scale bytes and codes byte-equal; the GEMM
consumes MSE-quantized weights unchanged."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import metrics as Mx
from oracle import nvfp4 as O
from oracle import scale_rules as S
from tests.gpu_util import Guarded, dev_bf16, host_bits, host_u8, log, need_gpu

pytestmark = pytest.mark.gpu
RULES = ("absmax", "four_over_six", "mse")


def _q():
    need_gpu()
    import quantized_gemm_nvfp4_amd as q
    return q


def gpu_quantize(bits, rule, g=None):
    q = _q()
    import torch
    R, C = bits.shape
    codes = Guarded((R, C // 2), torch.uint8)
    scales = Guarded((R, C // 16), torch.uint8)
    gt = torch.tensor([g], dtype=torch.float32, device="cuda:0") if g is not None else None
    out_g = gt if gt is not None else torch.empty(1, dtype=torch.float32, device="cuda:0")
    q.nvfp4_quantize(dev_bf16(bits), global_scale=gt, out=(codes.t, scales.t, out_g), rule=rule)
    torch.cuda.synchronize()
    assert codes.intact() and scales.intact(), "quantize wrote outside its outputs"
    return codes.t, scales.t, out_g


def assert_rule_equal(bits, rule, g=None, label="", rows=None):
    c, s, gg = gpu_quantize(bits, rule, g)
    gv = np.float32(gg.cpu().numpy()[0])
    sub = bits if rows is None else bits[rows]
    oc, os_, og = S.quantize(sub, rule=rule, g=gv if (rows is not None or g is not None) else None)
    if rows is None and g is None:
        assert gv.view(np.uint32) == np.float32(og).view(np.uint32), f"{label}: g {gv} != {og}"
    gc, gs = host_u8(c), host_u8(s)
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"{label} {rule}: {len(bad_s)} scale bytes differ, first at {bad_s[0]}"
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, f"{label} {rule}: {len(bad_c)} code bytes differ, first at {bad_c[0]}"
    return c, s, gg


@pytest.mark.parametrize("rule", RULES)
def test_hand_worked_blocks(golden, rule):
    g = golden("nvfp4_scale_rules_block.txt")
    for key in ("a", "b"):
        vals = np.array([float(t) for t in g[f"{key}_values"]], dtype=np.float32)[None, :]
        bits = F.bf16_bits(vals)
        c, s, _ = assert_rule_equal(bits, rule, g=1.0, label=f"block {key}")
        want = g[f"a_{rule}_scale"][0] if key == "a" else g["b_scale"][0]
        assert int(host_u8(s)[0, 0]) == int(want, 16)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("seed,shape,kw", [
    (31, (64, 512), dict(outlier_frac=0.01, outlier_mul=40)),
    (32, (33, 1024), dict(sigma=0.02, zero_frac=0.3)),
    (33, (8, 4096), dict(sigma=0.02, outlier_frac=0.002, outlier_mul=1000)),   # subnormal-scale blocks
])
def test_random_tensors(rule, seed, shape, kw):
    bits = workloads.random_bf16(seed, shape, **kw)
    assert_rule_equal(bits, rule, label=f"random {shape}")


def test_full_size_weight_sampled_rows():
    w_bits = workloads.decode_w()                    # [21504, 5376]
    rows = np.sort(np.random.default_rng(5).choice(w_bits.shape[0], 96, replace=False))
    for rule in ("four_over_six", "mse"):
        log(f"full-size W_up, rule {rule}: GPU quantize + oracle on 96 rows")
        assert_rule_equal(w_bits, rule, label="W_up", rows=rows)


def test_gemm_consumes_mse_weights():
    q = _q()
    import torch
    a_bits = workloads.random_bf16(41, (48, 2048))
    w_bits = workloads.random_bf16(42, (300, 2048), sigma=0.02, outlier_frac=0.005, outlier_mul=20)
    a = q.nvfp4_quantize(dev_bf16(a_bits))
    w = assert_rule_equal(w_bits, "mse", label="W")
    oa = O.quantize(a_bits)
    ow = S.quantize(w_bits, rule="mse")
    ref = O.gemm(*oa, *ow)
    for algo in (0, 1, 2, 3):
        a_in = a if algo != 2 else (a[0][:16], a[1][:16], a[2])
        y = q.nvfp4_gemm(a_in, w, algo=algo)
        torch.cuda.synchronize()
        yv = F.bf16_from_bits(host_bits(y)).astype(np.float64)
        ok, rl, rr = Mx.check_output(yv, ref if algo != 2 else ref[:16])
        log(f"gemm on MSE weights algo={algo}: rel_l2={rl:.3e} row_ratio={rr:.3e}")
        assert ok
