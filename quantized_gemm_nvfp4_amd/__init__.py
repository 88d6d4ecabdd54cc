"""Python binding of libnvfp4.so (C ABI in include/nvfp4.h).

Argument marshalling only: every step of quantization and matmul runs in the
library's HIP kernels.  Torch provides device memory and the current stream;
nothing here computes on the data.  If the library is missing or the HIP
runtime cannot load it, every call raises -- there is no CPU fallback.

Function names follow the C ABI:

* ``nvfp4_quantize(x, rule=...)``     -> (codes, scales, global_scale); rule absmax /
  four_over_six / mse
* ``nvfp4_gemm(a, w, algo=AUTO)``     -> bf16 [M, N]; a, w are the 3-tuples above
* ``nvfp4_gemm_amax(a, w)``           -> (bf16 [M, N], amax slots of the output)
* ``nvfp4_quantize_amax(x, slots)``   -> nvfp4_quantize(x) with max|x| from the slots
* ``nvfp4_gemm_w4a16(x, w)``          -> bf16 [M, N]; x bf16 (weight-only NVFP4)
* ``int4g_quantize(w, group=128)``    -> (q, scales_fp16)
* ``int4g_gemv(x, q, scales, ...)``   -> bf16 [M, N]
* ``int4g_asym_quantize(w)``          -> (q, scales_fp16, zeros_u8), zero-point INT4
* ``int4g_asym_gemv(x, q, s, z)``     -> bf16 [M, N]
* ``nvfp4_linear(x, w)``              -> quantize x and multiply (one kernel at M <= 2)
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

ALGO_AUTO, ALGO_TILED, ALGO_DECODE, ALGO_SIMPLE = 0, 1, 2, 3
STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_INVALID_ARG", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGNMENT",
          4: "NVFP4_ERR_UNSUPPORTED", 5: "NVFP4_ERR_HIP"}

# Every symbol include/nvfp4.h declares, with its ctypes signature.
_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, None
SIGNATURES = {
    "nvfp4_abi_version": ([], ctypes.c_int),
    "nvfp4_quantize_workspace_bytes": ([], ctypes.c_size_t),
    "nvfp4_quantize": ([_P, _I64, _I64, _P, _P, _P, _I, _P, _P], ctypes.c_int),
    "nvfp4_quantize_ex": ([_P, _I64, _I64, _P, _P, _P, _I, _I, _P, _P], ctypes.c_int),
    "nvfp4_quantize_noalloc": ([_P, _I64, _I64, _P, _P, _P, _I, _P], ctypes.c_int),
    "nvfp4_gemm": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "nvfp4_gemm_ex": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P], ctypes.c_int),
    "nvfp4_gemm_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "nvfp4_linear_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "nvfp4_linear": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "nvfp4_gemm_ws": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "nvfp4_gemm_amax_slots": ([_I64, _I64, _I64], ctypes.c_size_t),
    "nvfp4_gemm_amax": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "nvfp4_quantize_amax": ([_P, _I64, _I64, _P, _P, _P, _P, _I64, _P], ctypes.c_int),
    "nvfp4_gemm_w4a16": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "nvfp4_gemm_w4a16_ex": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P], ctypes.c_int),
    "int4g_quantize": ([_P, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "int4g_gemv": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "int4g_gemv_ex": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _P], ctypes.c_int),
    "int4g_asym_quantize": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "int4g_asym_gemv": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "int4g_asym_gemv_ex": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _P], ctypes.c_int),
    "nvfp4_quantize_lora_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "nvfp4_quantize_lora": ([_P, _I64, _I64, _P, _P, _P, _I, _P, _I64, _P, _P, _P], ctypes.c_int),
    "nvfp4_gemm_lora": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "nvfp4_gemm_lora_ex": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _I64, _I64, _I64, _I, _P], ctypes.c_int),
    "nvfp4_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "nvfp4_last_error": ([], ctypes.c_char_p),
}

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """The loaded library (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_gemm_nvfp4_amd.build` (or __graft_entry__.build())")
        # torch first: it loads the HIP runtime it ships with, and the
        # library then binds to that same runtime (loaded the other way
        # round, torch can find no device)
        _torch()
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(status):
    if status != 0:
        raise Nvfp4Error(status, lib().nvfp4_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


SCALE_RULES = {"absmax": 0, "four_over_six": 1, "mse": 2}


def nvfp4_quantize(x, global_scale=None, out=None, rule="absmax"):
    """NVFP4-quantize a bf16 [rows, cols] tensor (cols % 16 == 0).

    global_scale: optional fp32 device tensor [1] to use instead of the
    dynamic amax / 2688.  out: optional (codes, scales, global_scale) buffers.
    rule: block-scale selection, "absmax" (default), "four_over_six" or "mse".
    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16],
    global_scale fp32 [1]).
    """
    torch = _torch()
    _need(x, torch.bfloat16, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
        g = global_scale if global_scale is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, g = out
        if global_scale is not None and g is not global_scale:
            raise ValueError("pass the given global scale as out[2]")
    _need(codes, torch.uint8, (rows, cols // 2), "codes")
    _need(scales, torch.uint8, (rows, cols // 16), "scales")
    _need(g, torch.float32, (1,), "global_scale")
    use_given = 1 if global_scale is not None else 0
    ws = None
    if not use_given:
        ws = torch.empty(lib().nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device=x.device)
    if rule not in SCALE_RULES:
        raise ValueError(f"unknown scale rule {rule!r}; one of {sorted(SCALE_RULES)}")
    _check(lib().nvfp4_quantize_ex(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(g), use_given,
                                   SCALE_RULES[rule], _ptr(ws) if ws is not None else None, _stream(x)))
    return codes, scales, g


def nvfp4_gemm(a, w, algo=ALGO_AUTO, out=None, workspace=None):
    """bf16 [M, N] = g_a g_w dequant(A) . dequant(W)^T.

    a = (a_codes [M, K/2], a_scales [M, K/16], a_g [1]); w likewise with N rows.
    workspace: optional uint8 device tensor for the K split of the leftover
    tiles (nvfp4_gemm_workspace_bytes); when None one is taken from torch's
    allocator if the shape needs it.
    """
    torch = _torch()
    ac, as_, ag = a
    wc, ws, wg = w
    M, N = ac.shape[0], wc.shape[0]
    K = ac.shape[1] * 2
    _need(ac, torch.uint8, (M, K // 2), "a_codes")
    _need(as_, torch.uint8, (M, K // 16), "a_scales")
    _need(ag, torch.float32, (1,), "a_gscale")
    _need(wc, torch.uint8, (N, K // 2), "w_codes")
    _need(ws, torch.uint8, (N, K // 16), "w_scales")
    _need(wg, torch.float32, (1,), "w_gscale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=ac.device)
    _need(out, torch.bfloat16, (M, N), "out")
    if workspace is None:
        nbytes = lib().nvfp4_gemm_workspace_bytes(M, N, K)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=ac.device)
    if workspace is not None:
        _need(workspace, torch.uint8, None, "workspace")
    _check(lib().nvfp4_gemm_ws(_ptr(ac), _ptr(as_), _ptr(ag), _ptr(wc), _ptr(ws), _ptr(wg), _ptr(out),
                               M, N, K, int(algo), _ptr(workspace) if workspace is not None else None,
                               workspace.numel() if workspace is not None else 0, _stream(ac)))
    return out


def nvfp4_gemm_amax(a, w, out=None, workspace=None, slots=None):
    """nvfp4_gemm that also returns the amax slots of its output (uint32
    device tensor) for nvfp4_quantize_amax.  N % 16 == 0."""
    torch = _torch()
    ac, as_, ag = a
    wc, ws, wg = w
    M, N = ac.shape[0], wc.shape[0]
    K = ac.shape[1] * 2
    _need(ac, torch.uint8, (M, K // 2), "a_codes")
    _need(as_, torch.uint8, (M, K // 16), "a_scales")
    _need(ag, torch.float32, (1,), "a_gscale")
    _need(wc, torch.uint8, (N, K // 2), "w_codes")
    _need(ws, torch.uint8, (N, K // 16), "w_scales")
    _need(wg, torch.float32, (1,), "w_gscale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=ac.device)
    _need(out, torch.bfloat16, (M, N), "out")
    nslots = lib().nvfp4_gemm_amax_slots(M, N, K)
    if slots is None:
        slots = torch.empty(max(1, nslots), dtype=torch.int32, device=ac.device)
    _need(slots, torch.int32, None, "slots")
    if slots.numel() < nslots:
        raise ValueError(f"slots holds {slots.numel()} values, the call writes {nslots}")
    if workspace is None:
        nbytes = lib().nvfp4_gemm_workspace_bytes(M, N, K)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=ac.device)
    if workspace is not None:
        _need(workspace, torch.uint8, None, "workspace")
    _check(lib().nvfp4_gemm_amax(_ptr(ac), _ptr(as_), _ptr(ag), _ptr(wc), _ptr(ws), _ptr(wg), _ptr(out), M, N, K,
                                 _ptr(workspace) if workspace is not None else None,
                                 workspace.numel() if workspace is not None else 0, _ptr(slots), _stream(ac)))
    return out, slots[:nslots]


def nvfp4_quantize_amax(x, slots, out=None):
    """nvfp4_quantize(x) (absmax rule) with max|x| read from `slots` (as
    nvfp4_gemm_amax returns them for x) instead of a pass over x."""
    torch = _torch()
    _need(x, torch.bfloat16, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    _need(slots, torch.int32, None, "slots")
    rows, cols = x.shape
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, g = out
    _need(codes, torch.uint8, (rows, cols // 2), "codes")
    _need(scales, torch.uint8, (rows, cols // 16), "scales")
    _need(g, torch.float32, (1,), "global_scale")
    _check(lib().nvfp4_quantize_amax(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(g), _ptr(slots),
                                     slots.numel(), _stream(x)))
    return codes, scales, g


def nvfp4_gemm_w4a16(x, w, algo=ALGO_AUTO, out=None):
    """bf16 [M, N] = g_w x . dequant(W)^T with x bf16 [M, K] (weight-only)."""
    torch = _torch()
    wc, ws, wg = w
    _need(x, torch.bfloat16, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    N = wc.shape[0]
    _need(wc, torch.uint8, (N, K // 2), "w_codes")
    _need(ws, torch.uint8, (N, K // 16), "w_scales")
    _need(wg, torch.float32, (1,), "w_gscale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    _check(lib().nvfp4_gemm_w4a16_ex(_ptr(x), _ptr(wc), _ptr(ws), _ptr(wg), _ptr(out), M, N, K, algo, _stream(x)))
    return out


def nvfp4_linear(x, w, out=None, x_out=None, workspace=None):
    """Quantize bf16 x [M, K] (absmax rule, g from max|x|) and multiply by
    the NVFP4 weight w: bit-identical to nvfp4_gemm(nvfp4_quantize(x), w).

    One kernel does both when K % 128 == 0 and either M <= 2, K <= 8192 or
    3 <= M <= 16, M * K / 16 <= 3072.  x_out:
    optional (codes, scales, global_scale) buffers for x's NVFP4 form.
    Returns (out bf16 [M, N], (codes, scales, global_scale)).
    """
    torch = _torch()
    wc, ws, wg = w
    _need(x, torch.bfloat16, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    N = wc.shape[0]
    _need(wc, torch.uint8, (N, K // 2), "w_codes")
    _need(ws, torch.uint8, (N, K // 16), "w_scales")
    _need(wg, torch.float32, (1,), "w_gscale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    if x_out is None:
        x_out = (torch.empty((M, K // 2), dtype=torch.uint8, device=x.device),
                 torch.empty((M, K // 16), dtype=torch.uint8, device=x.device),
                 torch.empty(1, dtype=torch.float32, device=x.device))
    xc, xs, xg = x_out
    _need(xc, torch.uint8, (M, K // 2), "x_codes")
    _need(xs, torch.uint8, (M, K // 16), "x_scales")
    _need(xg, torch.float32, (1,), "x_gscale")
    if workspace is None:
        nbytes = lib().nvfp4_linear_workspace_bytes(M, N, K)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _need(workspace, torch.uint8, None, "workspace")
    _check(lib().nvfp4_linear(_ptr(x), _ptr(wc), _ptr(ws), _ptr(wg), _ptr(out), M, N, K, _ptr(xc), _ptr(xs),
                              _ptr(xg), _ptr(workspace) if workspace is not None else None,
                              workspace.numel() if workspace is not None else 0, _stream(x)))
    return out, x_out


def nvfp4_quantize_lora(x, lora_down, global_scale=None, out=None):
    """nvfp4_quantize (absmax) of x [rows, cols] plus T = x . lora_down^T.

    lora_down: bf16 [r, cols].  out: optional (codes, scales, global_scale,
    t) buffers.  Returns (codes, scales, global_scale, t fp32 [rows, r]).
    """
    torch = _torch()
    _need(x, torch.bfloat16, None, "x")
    if x.dim() != 2 or lora_down.dim() != 2:
        raise ValueError("x and lora_down must be 2-D")
    rows, cols = x.shape
    r = lora_down.shape[0]
    _need(lora_down, torch.bfloat16, (r, cols), "lora_down")
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
        g = global_scale if global_scale is not None else torch.empty(1, dtype=torch.float32, device=x.device)
        t = torch.empty((rows, r), dtype=torch.float32, device=x.device)
    else:
        codes, scales, g, t = out
        if global_scale is not None and g is not global_scale:
            raise ValueError("pass the given global scale as out[2]")
    _need(codes, torch.uint8, (rows, cols // 2), "codes")
    _need(scales, torch.uint8, (rows, cols // 16), "scales")
    _need(g, torch.float32, (1,), "global_scale")
    _need(t, torch.float32, (rows, r), "t")
    ws = torch.empty(lib().nvfp4_quantize_lora_workspace_bytes(rows, cols, r), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize_lora(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(g),
                                     1 if global_scale is not None else 0, _ptr(lora_down), r, _ptr(t), _ptr(ws),
                                     _stream(x)))
    return codes, scales, g, t


def nvfp4_gemm_lora(a, w, t, lora_up, algo=ALGO_AUTO, out=None):
    """nvfp4_gemm(a, w) + t . lora_up^T, rounded once to bf16.

    t: fp32 [M, r] (from nvfp4_quantize_lora); lora_up: bf16 [N, r].
    """
    torch = _torch()
    ac, as_, ag = a
    wc, ws, wg = w
    M, N = ac.shape[0], wc.shape[0]
    K = ac.shape[1] * 2
    r = t.shape[1] if t.dim() == 2 else -1
    _need(ac, torch.uint8, (M, K // 2), "a_codes")
    _need(as_, torch.uint8, (M, K // 16), "a_scales")
    _need(ag, torch.float32, (1,), "a_gscale")
    _need(wc, torch.uint8, (N, K // 2), "w_codes")
    _need(ws, torch.uint8, (N, K // 16), "w_scales")
    _need(wg, torch.float32, (1,), "w_gscale")
    _need(t, torch.float32, (M, r), "t")
    _need(lora_up, torch.bfloat16, (N, r), "lora_up")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=ac.device)
    _need(out, torch.bfloat16, (M, N), "out")
    _check(lib().nvfp4_gemm_lora_ex(_ptr(ac), _ptr(as_), _ptr(ag), _ptr(wc), _ptr(ws), _ptr(wg), _ptr(t),
                                    _ptr(lora_up), r, _ptr(out), M, N, K, int(algo), _stream(ac)))
    return out


def nvfp4_linear_lora(x, w, lora_down, lora_up, algo=ALGO_AUTO):
    """NVFP4 layer with a run-time low-rank branch: quantize x (computing
    T = x . lora_down^T in the same pass), then the GEMM with T . lora_up^T
    added before the bf16 rounding."""
    codes, scales, g, t = nvfp4_quantize_lora(x, lora_down)
    return nvfp4_gemm_lora((codes, scales, g), w, t, lora_up, algo=algo)


def int4g_quantize(w, group=128, out=None):
    """Symmetric INT4 per-group quantization of a bf16 [N, K] weight.
    Returns (q uint8 [N, K/2], scales fp16 [N, K/group])."""
    torch = _torch()
    _need(w, torch.bfloat16, None, "w")
    N, K = w.shape
    if out is None:
        q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
        s = torch.empty((N, K // group if group else 0), dtype=torch.float16, device=w.device)
    else:
        q, s = out
    _check(lib().int4g_quantize(_ptr(w), N, K, group, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def int4g_gemv(x, q, scales, group=128, algo=ALGO_AUTO, out=None):
    """W4A16: bf16 [M, N] = x . dequant(q, scales)^T."""
    torch = _torch()
    M, K = x.shape
    N = q.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(q, torch.uint8, (N, K // 2), "q")
    _need(scales, torch.float16, (N, K // group), "scales")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    _check(lib().int4g_gemv_ex(_ptr(x), _ptr(q), _ptr(scales), _ptr(out), M, N, K, group, int(algo),
                               _stream(x)))
    return out


def int4g_asym_quantize(w, group=128, out=None):
    """Asymmetric (zero-point) INT4 per-group quantization of a bf16 [N, K]
    weight.  Returns (q uint8 [N, K/2], scales fp16 [N, K/128], zeros uint8
    [N, K/128])."""
    torch = _torch()
    _need(w, torch.bfloat16, None, "w")
    N, K = w.shape
    if out is None:
        q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
        s = torch.empty((N, K // group), dtype=torch.float16, device=w.device)
        z = torch.empty((N, K // group), dtype=torch.uint8, device=w.device)
    else:
        q, s, z = out
    _need(q, torch.uint8, (N, K // 2), "q")
    _need(s, torch.float16, (N, K // group), "scales")
    _need(z, torch.uint8, (N, K // group), "zeros")
    _check(lib().int4g_asym_quantize(_ptr(w), N, K, group, _ptr(q), _ptr(s), _ptr(z), _stream(w)))
    return q, s, z


def int4g_asym_gemv(x, q, scales, zeros, group=128, algo=ALGO_AUTO, out=None):
    """bf16 [M, N] = x . (s16 (q - z))^T for the asymmetric INT4 weight."""
    torch = _torch()
    _need(x, torch.bfloat16, None, "x")
    M, K = x.shape
    N = q.shape[0]
    _need(q, torch.uint8, (N, K // 2), "q")
    _need(scales, torch.float16, (N, K // group), "scales")
    _need(zeros, torch.uint8, (N, K // group), "zeros")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    _check(lib().int4g_asym_gemv_ex(_ptr(x), _ptr(q), _ptr(scales), _ptr(zeros), _ptr(out), M, N, K, group, algo,
                                    _stream(x)))
    return out
