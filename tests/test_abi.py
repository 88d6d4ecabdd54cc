"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device.

The pointers passed here are never dereferenced: validation runs on the host
before any HIP call, so fake (but suitably aligned) addresses are safe."""
import ctypes
import os
import re

import pytest

import quantized_gemm_nvfp4_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, INVALID, SHAPE, ALIGN, UNSUP = 0, 1, 2, 3, 4
P = ctypes.c_void_p
A = P(0x10000)      # fake, 16-byte aligned, distinct addresses
B = P(0x20000)
C = P(0x30000)
D = P(0x40000)
E = P(0x50000)
F = P(0x60000)
G = P(0x70000)
ODD = P(0x10008)    # 8-byte aligned only


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z0-9_]+)\s*\(", text)) - {"defined"})


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "nvfp4_quantize" in names and "nvfp4_gemm" in names and "int4g_gemv" in names
    lib = q.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in nvfp4.h but not exported"
    assert set(names) == set(q.SIGNATURES), "binding signatures and header disagree"


def test_version_and_strings():
    lib = q.lib()
    assert lib.nvfp4_abi_version() == 1
    assert lib.nvfp4_quantize_workspace_bytes() == 4096
    assert lib.nvfp4_status_string(0) == b"ok"
    assert lib.nvfp4_status_string(3) == b"misaligned pointer"


def _err():
    return q.lib().nvfp4_last_error().decode()


def test_quantize_validation():
    lib = q.lib()
    f = lib.nvfp4_quantize
    assert f(None, 4, 32, B, C, D, 0, E, None) == INVALID and "x_bf16" in _err()
    assert f(A, 4, 32, B, C, D, 0, None, None) == INVALID and "workspace" in _err()
    assert f(A, -1, 32, B, C, D, 0, E, None) == INVALID
    assert f(A, 4, 24, B, C, D, 0, E, None) == SHAPE and "16" in _err()
    assert f(ODD, 4, 32, B, C, D, 0, E, None) == ALIGN
    assert f(A, 4, 32, ODD, C, D, 0, E, None) == ALIGN
    assert f(A, 4, 32, A, C, D, 0, E, None) == INVALID and "overlap" in _err()
    assert f(A, 4, 32, B, B, D, 0, E, None) == INVALID and "overlap" in _err()
    assert f(A, 1 << 40, 32, B, C, D, 0, E, None) == UNSUP
    # empty tensors: nothing to do, nothing enqueued
    assert f(A, 0, 32, B, C, D, 0, E, None) == OK
    assert f(A, 5, 0, B, C, D, 0, E, None) == OK
    assert _err() == ""
    # a given global scale needs no workspace
    assert f(A, 0, 32, B, C, D, 1, None, None) == OK


def test_quantize_ex_rule_validation():
    f = q.lib().nvfp4_quantize_ex
    assert f(A, 4, 32, B, C, D, 0, 3, E, None) == INVALID and "rule" in _err()
    assert f(A, 4, 32, B, C, D, 0, -1, E, None) == INVALID
    assert f(A, 4, 24, B, C, D, 0, 2, E, None) == SHAPE
    for rule in (0, 1, 2):
        assert f(A, 0, 32, B, C, D, 0, rule, E, None) == OK


def test_gemm_validation():
    f = q.lib().nvfp4_gemm_ex
    good = [A, B, C, D, E, F, G]
    assert f(*good, 32, 64, 120, 0, None) == SHAPE                 # K % 16
    assert f(*good, -3, 64, 128, 0, None) == INVALID
    assert f(None, *good[1:], 32, 64, 128, 0, None) == INVALID
    assert f(A, B, C, D, E, F, A, 32, 64, 128, 0, None) == INVALID  # out aliases a_codes
    assert f(A, B, C, D, E, F, ODD, 32, 64, 128, 0, None) == ALIGN
    assert f(A, B, P(0x30002), D, E, F, G, 32, 64, 128, 0, None) == ALIGN   # gscale 4-byte
    assert f(*good, 32, 64, 128, 9, None) == INVALID                # unknown algo
    assert f(*good, 32, 64, 144, q.ALGO_TILED, None) == UNSUP       # tiled needs K % 128
    assert f(*good, 17, 64, 128, q.ALGO_DECODE, None) == UNSUP      # decode needs M <= 16
    assert f(*good, 0, 64, 128, 0, None) == OK
    assert f(*good, 32, 0, 128, 0, None) == OK
    assert q.lib().nvfp4_gemm(*good, 32, 64, 120, None) == SHAPE
    ws = q.lib().nvfp4_gemm_ws
    W = P(0x100000)
    assert ws(*good, 32, 64, 128, 0, P(0x100010), 4096, None) == ALIGN         # workspace 256-byte aligned
    assert ws(*good, 32, 64, 128, 0, P(0x70000), 4096, None) == INVALID         # overlaps out
    assert ws(*good, 0, 64, 128, 0, W, 4096, None) == OK
    assert q.lib().nvfp4_gemm_workspace_bytes(16, 4096, 4096) == 0               # decode sizes never split
    assert q.lib().nvfp4_gemm_workspace_bytes(4096, 4096, 120) == 0              # K % 128


def test_amax_validation():
    lib = q.lib()
    assert lib.nvfp4_gemm_amax_slots(4096, 21504, 5376) == 16 * 84      # one per 256 x 256 tile
    assert lib.nvfp4_gemm_amax_slots(4096, 21504, 5376 + 16) == 1024    # simple kernel: a separate pass
    assert lib.nvfp4_gemm_amax_slots(8, 160, 256) == 1                  # decode: 1280 values, one partial
    assert lib.nvfp4_gemm_amax_slots(0, 160, 256) == 0
    good = [A, B, C, D, E, F, G]
    W = P(0x100000)
    S = P(0x200000)
    f = lib.nvfp4_gemm_amax
    assert f(*good, 32, 64, 128, W, 4096, None, None) == INVALID                 # no slots
    assert f(*good, 32, 72, 128, W, 4096, S, None) == SHAPE                      # N % 16
    assert f(*good, 32, 64, 128, W, 4096, P(0x200002), None) == ALIGN
    assert f(*good, 32, 64, 128, W, 4096, P(0x70000), None) == INVALID           # slots overlap out
    assert f(*good, 0, 64, 128, W, 4096, S, None) == OK
    g = lib.nvfp4_quantize_amax
    assert g(A, 4, 64, B, C, D, E, 0, None) == INVALID                           # nslots >= 1
    assert g(A, 4, 60, B, C, D, E, 4, None) == SHAPE
    assert g(A, 4, 64, B, C, D, None, 4, None) == INVALID
    assert g(A, 4, 64, B, C, D, P(0x50002), 4, None) == ALIGN
    assert g(A, 4, 64, A, C, D, E, 4, None) == INVALID                           # codes alias x
    assert g(A, 0, 64, B, C, D, E, 4, None) == OK


def test_decode_k_limit():
    # the weight-streaming kernels take K <= 2^24; beyond it an explicit
    # decode request is refused (before any device work)
    far = [P(k << 36) for k in range(1, 8)]      # fake, far apart: no overlap at this K
    K = (1 << 24) + 128
    assert q.lib().nvfp4_gemm_ex(*far, 4, 8, K, q.ALGO_DECODE, None) == UNSUP
    assert q.lib().int4g_gemv_ex(far[0], far[1], far[2], far[3], 4, 8, K, 128, q.ALGO_DECODE, None) == UNSUP


def test_nvfp4_tiled_k_limit():
    # the NVFP4 tiled kernel addresses a tile's rows with 32-bit offsets: an
    # explicit tiled request with K >= 2^24 is refused, no workspace is sized
    far = [P(k << 40) for k in range(1, 8)]
    K = 1 << 24
    assert q.lib().nvfp4_gemm_ex(*far, 32, 16, K, q.ALGO_TILED, None) == UNSUP
    assert "2^24" in _err()
    assert q.lib().nvfp4_gemm_workspace_bytes(4096, 4096, K) == 0
    assert q.lib().nvfp4_gemm_workspace_bytes(4096, 4096 + 256, K - 128) > 0


def test_int4_tiled_k_limit():
    # the INT4 tiled kernel addresses a tile's rows with 32-bit offsets: an
    # explicit tiled request with K >= 2^22 is refused before any device work
    far = [P(k << 38) for k in range(1, 5)]
    K = 1 << 22
    assert q.lib().int4g_gemv_ex(*far, 32, 8, K, 128, q.ALGO_TILED, None) == UNSUP
    assert "2^22" in _err()


def test_int4_validation():
    lib = q.lib()
    assert lib.int4g_quantize(A, 8, 256, 64, B, C, None) == UNSUP      # group must be 128
    assert lib.int4g_quantize(A, 8, 192, 128, B, C, None) == SHAPE     # K % group
    assert lib.int4g_quantize(A, 8, 256, 128, A, C, None) == INVALID   # q aliases w
    assert lib.int4g_quantize(A, 0, 256, 128, B, C, None) == OK
    g = lib.int4g_gemv_ex
    assert g(A, B, C, D, 4, 8, 256, 32, 0, None) == UNSUP
    assert g(A, B, C, D, 4, 8, 200, 128, 0, None) == SHAPE
    assert g(A, B, C, D, 17, 8, 256, 128, q.ALGO_DECODE, None) == UNSUP
    assert g(A, B, C, ODD, 4, 8, 256, 128, 0, None) == ALIGN
    assert g(A, B, C, D, 0, 8, 256, 128, 0, None) == OK
    assert lib.int4g_gemv(A, B, C, D, 4, 8, 256, 64, None) == UNSUP
    # out [M, N] past 2^40 elements: rejected before any range arithmetic
    big = (1 << 31) - 1
    assert g(A, B, C, D, big, big, 256, 128, 0, None) == UNSUP and "2^40" in _err()
    assert lib.int4g_asym_gemv_ex(A, B, C, D, E, big, big, 256, 128, 0, None) == UNSUP and "2^40" in _err()
    a = lib.int4g_asym_gemv_ex
    assert a(A, B, C, D, E, 4, 8, 256, 128, 9, None) == INVALID                       # unknown algo
    assert a(A, B, C, D, E, 3, 8, 256, 128, q.ALGO_DECODE, None) == UNSUP             # decode needs M <= 2
    far = [P(k << 40) for k in range(1, 6)]     # 1 TiB apart: the ranges of K = 2^22 cannot overlap
    assert a(*far, 64, 8, 1 << 22, 128, q.ALGO_TILED, None) == UNSUP and "2^22" in _err()   # tiled needs K < 2^22
    assert a(A, B, C, D, E, 0, 8, 256, 128, q.ALGO_TILED, None) == OK
    assert lib.nvfp4_gemm_w4a16_ex(A, B, C, D, E, big, big, 256, 0, None) == UNSUP and "2^40" in _err()


def test_w4a16_algo_validation():
    lib = q.lib()
    w = lib.nvfp4_gemm_w4a16_ex
    assert w(A, B, C, D, E, 4, 8, 256, 9, None) == INVALID                          # unknown algo
    assert w(A, B, C, D, E, 17, 8, 256, q.ALGO_DECODE, None) == UNSUP              # decode needs M <= 16
    assert w(A, B, C, D, E, 32, 8, 144, q.ALGO_TILED, None) == UNSUP               # tiled needs K % 128 == 0
    far = [P(k << 40) for k in range(1, 6)]     # 1 TiB apart: the ranges of K = 2^22 cannot overlap
    assert w(*far, 64, 8, 1 << 22, q.ALGO_TILED, None) == UNSUP and "2^22" in _err()
    assert w(A, B, C, D, E, 0, 8, 256, q.ALGO_TILED, None) == OK


def test_quantize_noalloc_validation():
    lib = q.lib()
    f = lib.nvfp4_quantize_noalloc
    # x, rows, cols, codes, scales, g, use_given, stream
    assert f(None, 4, 32, B, C, D, 0, None) == INVALID and "x_bf16" in _err()
    assert f(A, 4, 24, B, C, D, 0, None) == SHAPE
    assert f(A, 4, 32, ODD, C, D, 0, None) == ALIGN
    assert f(A, 4, 32, A, C, D, 0, None) == INVALID and "overlap" in _err()
    assert f(A, -1, 32, B, C, D, 0, None) == INVALID
    assert f(A, 1 << 30, 1 << 30, B, C, D, 0, None) == UNSUP
    assert f(A, 0, 32, B, C, D, 0, None) == OK


def test_linear_validation():
    lib = q.lib()
    f = lib.nvfp4_linear
    H, W = P(0x80000), P(0x100000)
    # x, w_codes, w_scales, w_g, out, M, N, K, x_codes, x_scales, x_g, workspace, bytes, stream
    good = [A, B, C, D, E]
    xo = [F, G, H]
    assert f(None, B, C, D, E, 1, 64, 128, *xo, None, 0, None) == INVALID and "x_bf16" in _err()
    assert f(*good, 1, 64, 128, None, G, H, None, 0, None) == INVALID and "x_codes" in _err()
    assert f(*good, 1, 64, 0, *xo, None, 0, None) == SHAPE                      # K must be positive
    assert f(*good, 1, 64, 120, *xo, None, 0, None) == SHAPE                    # K % 16
    assert f(*good, -1, 64, 128, *xo, None, 0, None) == INVALID
    assert f(A, B, C, D, ODD, 1, 64, 128, *xo, None, 0, None) == ALIGN
    assert f(*good, 1, 64, 128, F, G, P(0x80002), None, 0, None) == ALIGN     # x_g 4-byte
    assert f(*good, 1, 64, 128, A, G, H, None, 0, None) == INVALID and "overlap" in _err()
    assert f(*good, 1, 64, 128, F, G, E, None, 0, None) == INVALID and "overlap" in _err()
    # one-kernel shapes need no workspace; the others need the quantizer's
    assert lib.nvfp4_linear_workspace_bytes(1, 21504, 5376) == 0
    assert lib.nvfp4_linear_workspace_bytes(2, 64, 8192) == 0
    assert lib.nvfp4_linear_workspace_bytes(1, 64, 8192 + 128) == 4096
    assert lib.nvfp4_linear_workspace_bytes(3, 64, 128) == 0
    assert lib.nvfp4_linear_workspace_bytes(16, 64, 3072) == 0                 # M K / 16 = 3072
    assert lib.nvfp4_linear_workspace_bytes(16, 64, 3072 + 128) == 4096
    assert lib.nvfp4_linear_workspace_bytes(17, 64, 128) == 4096
    assert lib.nvfp4_linear_workspace_bytes(2, 64, 48) == 4096
    assert lib.nvfp4_linear_workspace_bytes(4096, 4096, 4096) >= 4096
    assert f(*good, 17, 64, 128, *xo, None, 0, None) == INVALID and "workspace" in _err()
    assert f(*good, 17, 64, 128, *xo, P(0x100010), 4096, None) == ALIGN
    assert f(*good, 17, 64, 128, *xo, W, 4095, None) == INVALID
    assert f(*good, 0, 64, 128, *xo, None, 0, None) == OK
    assert f(*good, 1 << 30, 1 << 30, 128, *xo, None, 0, None) == UNSUP


def test_lora_workspace_size():
    f = q.lib().nvfp4_quantize_lora_workspace_bytes
    # one K slice: only the 1024 partial maxima
    assert f(20000, 3072, 32) == 4096
    assert f(8, 128, 32) == 4096
    # decode row (1 row group): min(1024, 168 steps / 8) = 21 slices of partial T
    assert f(1, 5376, 32) == 4096 + 21 * 1 * 32 * 4
    # 256 row groups: 1024 / 256 = 4 slices
    assert f(4096, 3072, 32) == 4096 + 4 * 4096 * 32 * 4
    assert f(-1, 128, 8) == 0 and f(4, 128, 256) == 0


def test_lora_validation():
    lib = q.lib()
    f = lib.nvfp4_quantize_lora
    # x, rows, cols, codes, scales, g, use_given, lora_down, r, t, workspace, stream
    assert f(A, 4, 32, B, C, D, 0, E, 12, F, G, None) == UNSUP and "rank" in _err()     # r % 8
    assert f(A, 4, 32, B, C, D, 0, E, 0, F, G, None) == UNSUP
    assert f(A, 4, 32, B, C, D, 0, E, 136, F, G, None) == UNSUP                         # r > 128
    assert f(A, 4, 24, B, C, D, 0, E, 16, F, G, None) == SHAPE
    assert f(A, 4, 32, B, C, D, 0, E, 16, F, None, None) == INVALID and "workspace" in _err()
    assert f(A, 4, 32, B, C, D, 1, E, 16, F, None, None) == INVALID   # always needs the workspace
    assert f(A, 4, 32, B, C, D, 0, None, 16, F, G, None) == INVALID
    assert f(A, 4, 32, B, C, D, 0, E, 16, ODD, G, None) == ALIGN
    assert f(A, 4, 32, B, C, D, 0, E, 16, A, G, None) == INVALID and "overlap" in _err()  # t aliases x
    assert f(A, 0, 32, B, C, D, 0, E, 16, F, G, None) == OK
    g = lib.nvfp4_gemm_lora_ex
    # a_codes, a_scales, a_g, w_codes, w_scales, w_g, t, up, r, out, M, N, K, algo, stream
    T, U, O = P(0x80000), P(0x90000), P(0xA0000)
    assert g(A, B, C, D, E, F, T, U, 20, O, 4, 8, 128, 0, None) == UNSUP                 # r % 8
    assert g(A, B, C, D, E, F, None, U, 16, O, 4, 8, 128, 0, None) == INVALID
    assert g(A, B, C, D, E, F, T, U, 16, O, 4, 8, 120, 0, None) == SHAPE
    assert g(A, B, C, D, E, F, T, U, 16, T, 4, 8, 128, 0, None) == INVALID and "overlap" in _err()
    assert g(A, B, C, D, E, F, ODD, U, 16, O, 4, 8, 128, 0, None) == ALIGN
    assert g(A, B, C, D, E, F, T, U, 16, O, 17, 8, 128, q.ALGO_DECODE, None) == UNSUP
    assert g(A, B, C, D, E, F, T, U, 16, O, 0, 8, 128, 0, None) == OK
    assert lib.nvfp4_gemm_lora(A, B, C, D, E, F, T, U, 4, O, 4, 8, 128, None) == UNSUP


def test_error_text_is_thread_local():
    import threading
    lib = q.lib()
    assert lib.nvfp4_quantize(A, 4, 24, B, C, D, 0, E, None) == SHAPE
    seen = {}

    def other():
        seen["msg"] = lib.nvfp4_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "16" in _err()


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        q.nvfp4_quantize(torch.zeros((2, 32), dtype=torch.bfloat16))
