"""Seeded synthetic inputs for the NVFP4 / INT4 hot path.

This module only draws random numbers and rounds them to bf16 (a plain
library cast); it holds none of the quantization or GEMM arithmetic.  Both
the CPU oracle's tests and the GPU path's tests and benchmark take their
inputs from here.

Every tensor is drawn from ``numpy.random.default_rng([workload, tensor_id])``
as float32 standard normals times sigma (float32 multiply), with any outlier
scaling applied in float32, then rounded to bf16 with torch's CPU cast
(round-to-nearest-even).  Tensors are returned as numpy uint16 arrays of bf16
bit patterns.

Workloads (shapes and distributions stand in for the pages' workloads: a
dense decoder MLP on the Gemma-4 page and the diffusion-transformer linears
on the Flux2 / Wan 2.1 page; the pages name no public dataset):

* ``tiny``    -- W4A4 linear: A [16, 256] ~ N(0, 1), W [256, 256] ~ N(0, 0.02).
* ``decode``  -- x [16, 5376] ~ N(0, 1) with 5 of 5376 channels (0.1%) x20;
                 W_up [21504, 5376] ~ N(0, 0.02).  M = 1 and 4 use the first rows.
* ``prefill`` -- x_up [4096, 5376] ~ N(0, 1); W_up (the decode weight);
                 W_down [5376, 21504] ~ N(0, 0.02).
* ``dit``     -- W_qkv [9216, 3072], W_up [12288, 3072], W_down [3072, 12288]
                 ~ N(0, 0.02); x_t [4096, 3072] ~ N(0, 1) for steps t = 0..3.
* ``int4``    -- W [28672, 8192] ~ N(0, 0.02) with a Bernoulli(0.005) mask of
                 entries x10; x [2048, 8192] ~ N(0, 1).  M = 1, 16 use the first rows.
"""
import functools

import numpy as np

WORKLOAD_IDS = {"tiny": 0, "decode": 2, "prefill": 3, "dit": 4, "int4": 5, "lora": 6}

SHAPES = {
    "tiny": {"M": 16, "N": 256, "K": 256},
    "decode": {"M": (1, 4, 16), "N": 21504, "K": 5376},
    "prefill": {"M": 4096, "up": (21504, 5376), "down": (5376, 21504)},
    "dit": {"M": 4096, "qkv": (9216, 3072), "up": (12288, 3072), "down": (3072, 12288), "steps": 4},
    "int4": {"M": (1, 16, 2048), "N": 28672, "K": 8192, "group": 128},
    "lora": {"M": 4096, "qkv": (9216, 3072), "rank": 32},
}


def _to_bf16_bits(a32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(workload, tensor_id, shape, sigma=1.0, chunk_rows=None):
    """bf16 bits of N(0, sigma^2) draws from rng([workload, tensor_id])."""
    rng = np.random.default_rng([WORKLOAD_IDS[workload], tensor_id])
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return _to_bf16_bits(a)


@functools.lru_cache(maxsize=None)
def tiny():
    a = normal_bf16("tiny", 0, (16, 256))
    w = normal_bf16("tiny", 1, (256, 256), 0.02)
    return a, w


@functools.lru_cache(maxsize=None)
def decode_x():
    """x [16, 5376]: N(0,1) with round(0.001 * 5376) = 5 channels scaled x20
    (the same columns in every row), chosen without replacement."""
    rng = np.random.default_rng([WORKLOAD_IDS["decode"], 0])
    x = rng.standard_normal((16, 5376), dtype=np.float32)
    cols = np.random.default_rng([WORKLOAD_IDS["decode"], 1]).choice(5376, 5, replace=False)
    x[:, cols] *= np.float32(20.0)
    return _to_bf16_bits(x), np.sort(cols)


@functools.lru_cache(maxsize=None)
def decode_w():
    return normal_bf16("decode", 2, (21504, 5376), 0.02)


@functools.lru_cache(maxsize=None)
def prefill():
    x_up = normal_bf16("prefill", 0, (4096, 5376))
    w_down = normal_bf16("prefill", 1, (5376, 21504), 0.02)
    return x_up, decode_w(), w_down


@functools.lru_cache(maxsize=None)
def dit_weights():
    return (normal_bf16("dit", 0, (9216, 3072), 0.02),
            normal_bf16("dit", 1, (12288, 3072), 0.02),
            normal_bf16("dit", 2, (3072, 12288), 0.02))


@functools.lru_cache(maxsize=None)
def dit_x(step):
    return normal_bf16("dit", 10 + step, (4096, 3072))


@functools.lru_cache(maxsize=None)
def int4_w():
    """W [28672, 8192] ~ N(0, 0.02), Bernoulli(0.005) entries x10."""
    shape = (28672, 8192)
    a = np.random.default_rng([WORKLOAD_IDS["int4"], 0]).standard_normal(shape, dtype=np.float32)
    a *= np.float32(0.02)
    mask = np.random.default_rng([WORKLOAD_IDS["int4"], 1]).random(shape, dtype=np.float32) < np.float32(0.005)
    a[mask] *= np.float32(10.0)
    del mask
    return _to_bf16_bits(a)


@functools.lru_cache(maxsize=None)
def int4_x():
    return normal_bf16("int4", 2, (2048, 8192))


@functools.lru_cache(maxsize=None)
def dit_lora(rank=32):
    """Low-rank factors on the qkv projection [9216, 3072] of the diffusion
    stack: L_down bf16 [rank, 3072] and L_up bf16 [9216, rank], both
    ~ N(0, 0.02) (a trained adapter: L_up is not the zero initialization)."""
    return (normal_bf16("lora", rank, (rank, 3072), 0.02),
            normal_bf16("lora", 1000 + rank, (9216, rank), 0.02))


def random_f32(seed, shape, sigma=1.0):
    """Seeded fp32 tensor ~ N(0, sigma^2) with full 24-bit mantissas."""
    rng = np.random.default_rng([101, seed])
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


def random_bf16(seed, shape, sigma=1.0, outlier_frac=0.0, outlier_mul=1.0, zero_frac=0.0):
    """Generic seeded bf16 tensor for parity cases outside the named workloads
    (ragged shapes, degenerate blocks): N(0, sigma^2), optional outliers and
    exact zeros."""
    rng = np.random.default_rng([100, seed])
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    if outlier_frac:
        m = rng.random(shape) < outlier_frac
        a[m] *= np.float32(outlier_mul)
    if zero_frac:
        a[rng.random(shape) < zero_frac] = 0.0
    return _to_bf16_bits(a)


def blocks_at_scale_ratio(seed, g, nblk, log2_lo, log2_hi, cols=1024):
    """bf16 bits of nblk 16-value blocks (rows of `cols` values) whose
    largest magnitude is about r * 6 * g, log2 r uniform in [log2_lo,
    log2_hi]: one element of each block at +-that magnitude, the others
    uniform in [-1, 1] times it."""
    rng = np.random.default_rng([101, seed])
    amax = 2.0 ** rng.uniform(log2_lo, log2_hi, size=nblk) * 6.0 * float(g)
    u = rng.uniform(-1.0, 1.0, size=(nblk, 16))
    u[:, 0] = np.where(rng.random(nblk) < 0.5, 1.0, -1.0)
    return _to_bf16_bits((u * amax[:, None]).astype(np.float32).reshape(-1, cols))
