"""NVFP4 block-scale selection rules: absmax, four-over-six, MSE -- plain numpy.

Test infrastructure only (see ``oracle/__init__.py``).

What the page fixes ("Tu pipeline NVFP4 ...", section 2, the table of scale
algorithms): the scale of a 16-value block can be

* **absmax** -- the block's largest magnitude sets the scale (it maps to the
  largest E2M1 value, 6).  This is ``nvfp4.quantize``.
* **MSE** -- several candidate scales are tried and the one with the smallest
  reconstruction error of the block is kept.
* **four-over-six** -- each block picks, of the two possible largest values 4
  and 6, the one that reconstructs the block with less error.

Readings taken where the page is silent (each listed in the design notes):

1. The per-tensor scale g and all arithmetic of ``nvfp4.quantize`` are kept;
   a rule only changes which E4M3 scale byte a block stores.  The codes are
   then computed from that stored scale exactly as for absmax
   (d = fl32(s * g), y = fl32(x / d), E2M1 nearest-even).
2. Reconstruction error of a block under a candidate scale: fp32 arithmetic
   with one rounding per step, x_hat_j = fl32(v_j * d) (v_j the signed E2M1
   value of element j's code), e_j = fl32(x_j - x_hat_j), and
   err = sum over j = 0..15, in that order, of fl32(e_j * e_j), accumulated
   in fp32 from 0.  The decision is taken in this precision on both sides of
   the parity check.
3. Four-over-six candidates: s6 = E4M3(fl32(fl32(amax_b / 6) / g)) and
   s4 = E4M3(fl32(fl32(amax_b / 4) / g)) (both saturating at 448); s4 is
   kept only if its error is strictly smaller.
4. MSE candidates: the E4M3 codes within 8 codes (one binade) of the absmax
   scale's code c6, visited in the order c6, c6 - 1, c6 + 1, c6 - 2, ...,
   c6 + 8, restricted to codes 1..0x7E; a candidate replaces the current best
   only with a strictly smaller error.  The window contains the
   four-over-six candidate (its code is at most 5 above c6), so the MSE
   error never exceeds the four-over-six error, which never exceeds absmax.

Parity: pinned by tests/test_oracle_scale_rules.py -- a hand-worked block
(tests/golden/nvfp4_scale_rules_block.txt) where max->4 reconstructs exactly
and absmax does not, blocks built to be exact under a known in-window scale,
a brute-force fp64 search over the window, and the error ordering
absmax >= four-over-six >= MSE.
"""
import numpy as np

from . import formats as F
from . import nvfp4 as Q

RULES = ("absmax", "four_over_six", "mse")
MSE_WINDOW = 8                   # E4M3 codes either side of the absmax scale
E4M3_MAX_CODE = 0x7E


def _block_scale_code(amax_b, g, top):
    """E4M3 byte of fl32(fl32(amax_b / top) / g) (0 when g == 0)."""
    if g == 0:
        return np.zeros(amax_b.shape, dtype=np.uint8)
    s_raw = ((amax_b / np.float32(top)).astype(np.float32) / g).astype(np.float32)
    return F.e4m3_encode_nonneg(s_raw).astype(np.uint8)


def _codes_for_scale(blocks, s_code, g):
    """Element codes [..., 16] and d = fl32(s * g) [...] for given scale bytes."""
    s_val = F.e4m3_decode(s_code).astype(np.float32)
    d = (s_val * g).astype(np.float32)
    d_b = np.broadcast_to(d[..., None], blocks.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(d_b != 0, blocks / np.where(d_b != 0, d_b, np.float32(1)), np.float32(0))
    y = y.astype(np.float32)
    mag = F.e2m1_encode_magnitude(np.abs(y))
    sign = np.signbit(blocks).astype(np.uint8)
    return ((sign << 3) | mag).astype(np.uint8), d


def block_error(blocks, codes, d):
    """fp32 reconstruction error of each block (reading 2), shape blocks[:-1]."""
    v = F.e2m1_decode(codes).astype(np.float32)              # signed, exact
    xhat = (v * d[..., None]).astype(np.float32)
    e = (blocks - xhat).astype(np.float32)
    sq = (e * e).astype(np.float32)
    acc = np.zeros(blocks.shape[:-1], dtype=np.float32)
    for j in range(Q.BLOCK):
        acc = (acc + sq[..., j]).astype(np.float32)
    return acc


def choose_scales(blocks, g, rule):
    """E4M3 scale byte per block [R, C/16] under ``rule`` (readings 3-4)."""
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule!r}")
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    c6 = _block_scale_code(amax_b, g, 6.0)
    if rule == "absmax":
        return c6
    codes6, d6 = _codes_for_scale(blocks, c6, g)
    best_c, best_e = c6.copy(), block_error(blocks, codes6, d6)
    if rule == "four_over_six":
        c4 = _block_scale_code(amax_b, g, 4.0)
        codes4, d4 = _codes_for_scale(blocks, c4, g)
        e4 = block_error(blocks, codes4, d4)
        take = e4 < best_e
        return np.where(take, c4, best_c).astype(np.uint8)
    for step in range(1, MSE_WINDOW + 1):
        for k in (-step, step):
            c = c6.astype(np.int32) + k
            valid = (c >= 1) & (c <= E4M3_MAX_CODE)
            cc = np.where(valid, c, 1).astype(np.uint8)
            codes_k, d_k = _codes_for_scale(blocks, cc, g)
            e_k = block_error(blocks, codes_k, d_k)
            take = valid & (e_k < best_e)
            best_c = np.where(take, cc, best_c).astype(np.uint8)
            best_e = np.where(take, e_k, best_e).astype(np.float32)
    return best_c


def quantize(x, rule="absmax", g=None):
    """NVFP4-quantize X [R, C] with the block-scale rule ``rule``.

    Same inputs and outputs as ``nvfp4.quantize`` (codes, scales, g); with
    rule="absmax" the result is identical to it.
    """
    xf = Q._as_bf16_values(x)
    if xf.ndim != 2 or xf.shape[1] % Q.BLOCK:
        raise ValueError("quantize expects a 2-D array with C % 16 == 0")
    R, C = xf.shape
    g = Q.global_scale(xf) if g is None else np.float32(g)
    blocks = xf.reshape(R, C // Q.BLOCK, Q.BLOCK)
    s_code = choose_scales(blocks, g, rule)
    code, _ = _codes_for_scale(blocks, s_code, g)
    code = code.reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code.astype(np.uint8), np.float32(g)


def reconstruction_error(x, packed, scales, g):
    """Per-block fp32 error (reading 2) of an encoded matrix, [R, C/16]."""
    xf = Q._as_bf16_values(x)
    R, C = xf.shape
    blocks = xf.reshape(R, C // Q.BLOCK, Q.BLOCK)
    codes = Q.unpack_codes(packed).reshape(R, C // Q.BLOCK, Q.BLOCK)
    d = (F.e4m3_decode(np.asarray(scales, dtype=np.uint8)).astype(np.float32) * np.float32(g)).astype(np.float32)
    return block_error(blocks, codes, d)
