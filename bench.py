"""Benchmark of the NVFP4 hot path on one MI355X.

One step = the prefill chain on the M = 4096 dense-decoder MLP:
    quantize x_up [4096, 5376]  ->  GEMM up   (x W_up^T,   W_up   [21504, 5376])
    quantize h    [4096, 21504] ->  GEMM down (h W_down^T, W_down [5376, 21504])
with dynamic per-call activation quantization (the weights are quantized once,
before timing).  `value` is 2 * (M*N*K for both GEMMs) / step time, in TFLOP/s,
activation quantization included.

The same run also measures, on their own timed loops, the decode GEMV at
M = 1 (GB/s of algorithmic bytes, rotating 16 weight copies so every call
misses the 256 MB last-level cache), the DiT linear stack over 4 steps, and
the INT4 per-group W4A16 path (M = 1 and 16 in GB/s, M = 2048 in TFLOP/s).

`roofline` reports the tiled GEMM kernel: algorithmic FLOPs per launch over
its average launch time, measured with events on the launch stream inside
the timed region, against the fp16/bf16 dense MFMA peak (2.5 PFLOP/s).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

`peaks` holds the measured denominators (peak/peak.hip: a dense fp16 MFMA
loop, a 1 GiB read, a plain read of the decode weight's bytes per call), and
the roofline and decode entries carry their fractions of those as well.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
                       [--no-cpu-baseline] [--copy-calibration]
       python bench.py --decode-traffic            (for rocprofv3 --pmc runs)
       python bench.py --traffic-from F W | --decode-traffic-from F W
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s incl. act quant (M=4096) + decode GB/s (M=1); % roofline"
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_tiled_prefill.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


class Timer:
    """Elapsed-time events recorded on the launch stream.

    They are created with hipEventDisableSystemFence: a default event record
    ends with a system-scope release (L2 writeback and invalidation), which on
    this GPU left the next kernel idle for ~10 us, so events between the
    calls of a step would lengthen the step they measure.  These events are
    read only after a host synchronize, for timestamps."""
    FLAGS = 0x20000000     # hipEventDisableSystemFence
    _hip = None

    def __init__(self, torch, stream):
        import ctypes
        if Timer._hip is None:
            torch.cuda.init()
            hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            Timer._hip = hip
        self.ctypes = ctypes
        self.stream = stream
        self.pairs = []

    def _check(self, err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed with HIP error {err}")

    def _event(self):
        e = self.ctypes.c_void_p()
        self._check(Timer._hip.hipEventCreateWithFlags(self.ctypes.byref(e), Timer.FLAGS), "hipEventCreateWithFlags")
        self._check(Timer._hip.hipEventRecord(e, self.stream), "hipEventRecord")
        return e

    def start(self):
        return self._event()

    def stop(self, s):
        self.pairs.append((s, self._event()))

    def ms(self):
        """Durations in ms (call after a synchronize); releases the events."""
        out = []
        for s, e in self.pairs:
            v = self.ctypes.c_float()
            self._check(Timer._hip.hipEventElapsedTime(self.ctypes.byref(v), s, e), "hipEventElapsedTime")
            out.append(v.value)
            Timer._hip.hipEventDestroy(s)
            Timer._hip.hipEventDestroy(e)
        self.pairs = []
        return out


DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode.json")
DECODE_SOURCES = ("gemm_decode.hip", "int4_gemm.hip", "int4_asym.hip", "quant_block.h", "common.h")


def kernel_source_hash(files=("gemm_tiled.hip", "common.h")):
    """Hash of kernel sources with comments and whitespace removed, so that
    counters taken on a build stay valid across comment-only edits."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_gemm_nvfp4_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"//[^\n]*", "", src)
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        h.update(re.sub(r"\s+", " ", src).strip().encode())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per tiled-GEMM launch from committed rocprofv3 counters, or
    None if they were taken on a different version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def summarize_traffic(fetch_csv, write_csv):
    """Write TRAFFIC_FILE from the counter CSVs of two rocprofv3 --pmc runs
    of `bench.py --steps 5 --warmup 2 --no-extras --no-cpu-baseline
    --copy-calibration` (FETCH_SIZE, then WRITE_SIZE).  Counter units are
    converted to bytes with what the same counter reads for the 1 GiB device
    copies of the run; medians over the launches of each GEMM (up: the
    instance with the amax epilogue, down: the plain one; a reduce kernel
    belongs to the GEMM dispatched before it)."""
    import csv

    def load(path, counter):
        rows = sorted((r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter),
                      key=lambda r: int(r["Dispatch_Id"]))
        vals = {"up": [], "down": [], "reduce_up": [], "reduce_down": [], "copy": []}
        last = None
        for r in rows:
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "nvfp4_gemm_tiled_kernel<4, false, true" in name:
                last = "up"
                vals["up"].append(v)
            elif "nvfp4_gemm_tiled_kernel<4, false, false" in name:
                last = "down"
                vals["down"].append(v)
            elif "nvfp4_gemm_tiled_reduce_kernel" in name and last:
                vals["reduce_" + last].append(v)
            elif "copyBuffer" in name:
                vals["copy"].append(v)
        return {k: float(np.median(v)) if v else 0.0 for k, v in vals.items()}

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_bytes = 1 << 30
    fu, wu = copy_bytes / fetch["copy"], copy_bytes / write["copy"]
    M = 4096
    shapes = {"up": (21504, 5376), "down": (5376, 21504)}
    per = {}
    for k, (N, K) in shapes.items():
        alg = M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + M * N * 2 + 8
        per[k] = {"gemm_fetch_bytes": round(fetch[k] * fu), "gemm_write_bytes": round(write[k] * wu),
                  "reduce_fetch_bytes": round(fetch["reduce_" + k] * fu),
                  "reduce_write_bytes": round(write["reduce_" + k] * wu), "algorithmic_bytes": alg,
                  "gemm_traffic_over_algorithmic": round((fetch[k] * fu + write[k] * wu) / alg, 2)}
    cmd = "rocprofv3 --pmc {c} --output-format csv -d <dir> -o {o} -- python3 -u bench.py --steps 5 --warmup 2 " \
          "--no-extras --no-cpu-baseline --copy-calibration"
    out = {
        "kernel": "nvfp4_gemm_tiled_kernel<4, false, true, true> (up, with the amax epilogue) and "
                  "<4, false, false, true> (down); the last argument: scales copied four K stages at a time",
        "workload": "prefill up (M=4096, N=21504, K=5376) and down (M=4096, N=5376, K=21504) GEMMs, with the "
                    "last-round K split, as bench.py times them",
        "kernel_source_hash": kernel_source_hash(),
        "bytes_per_launch": round(np.mean([per[k]["gemm_fetch_bytes"] + per[k]["gemm_write_bytes"] for k in per])),
        "per_shape": per,
        "calibration": {"copy_bytes": copy_bytes, "FETCH_SIZE_per_copy": fetch["copy"],
                        "WRITE_SIZE_per_copy": write["copy"], "bytes_per_FETCH_unit": fu, "bytes_per_WRITE_unit": wu},
        "commands": [cmd.format(c="FETCH_SIZE", o="fetch"), cmd.format(c="WRITE_SIZE", o="write"),
                     "python3 bench.py --traffic-from <dir>/fetch_counter_collection.csv "
                     "<dir>/write_counter_collection.csv"],
        "note": "Counter values scaled by what the same counters read for a 1 GiB device copy (torch copy_, the "
                "__amd_rocclr_copyBuffer dispatches in the same run); medians over the launches of each shape. "
                "bytes_per_launch is the mean of the up and down GEMM kernels (fetch + write), matching "
                "roofline.achieved, which averages the two launches.",
        "hash_note": "sha256 (first 16 hex digits) of gemm_tiled.hip + common.h with comments and whitespace "
                     "removed, as bench.py computes it",
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    return out


# The decode-sized kernels whose HBM bytes per call bench.py --decode-traffic
# exposes to rocprofv3 --pmc: (name, weight, M), launched in this order.
DECODE_TRAFFIC = [
    ("nvfp4_w4a4_M1", "nvfp4", 1), ("nvfp4_w4a4_M2", "nvfp4", 2), ("nvfp4_w4a4_M4", "nvfp4", 4),
    ("nvfp4_w4a4_M16", "nvfp4", 16), ("nvfp4_linear_M1", "nvfp4", 1), ("nvfp4_linear_M2", "nvfp4", 2),
    ("nvfp4_linear_M4", "nvfp4", 4),
    ("nvfp4_w4a16_M1", "nvfp4", 1), ("nvfp4_w4a16_M2", "nvfp4", 2), ("nvfp4_w4a16_M4", "nvfp4", 4),
    ("nvfp4_w4a16_M16", "nvfp4", 16), ("int4_M1", "int4", 1), ("int4_M4", "int4", 4), ("int4_M16", "int4", 16),
    ("int4_asym_M1", "int4_asym", 1)]
DECODE_TRAFFIC_LAUNCHES = 6


def decode_alg_bytes(name, M):
    """Algorithmic bytes of one call: weight codes + scales (+ zeros) + the
    activation as the call takes it + the bf16 output."""
    if name.startswith("int4"):
        N, K = 28672, 8192
        per_group = 3 if name.startswith("int4_asym") else 2
        return N * K // 2 + N * (K // 128) * per_group + M * K * 2 + M * N * 2
    N, K = 21504, 5376
    w = N * K // 2 + N * K // 16 + 4 + M * N * 2
    if "w4a4" in name:
        return w + M * K // 2 + M * K // 16 + 4
    if "linear" in name:   # reads bf16 x, writes its codes, scales and g
        return w + M * K * 2 + M * K // 2 + M * K // 16 + 4
    return w + M * K * 2


def run_decode_traffic(torch, q, launches=DECODE_TRAFFIC_LAUNCHES):
    """For rocprofv3 --pmc runs: after three 1 GiB device copies (the counter
    calibration), each DECODE_TRAFFIC kernel is launched `launches` times in
    order, each launch on the next of several weight copies (~1 GB in all per
    weight), so every call reads its weight from HBM."""
    import workloads
    xn, _ = workloads.decode_x()
    wn = q.nvfp4_quantize(dev_bf16(torch, workloads.decode_w()))
    rot_n = [tuple(t.clone() for t in wn) for _ in range(16)]
    del wn
    wi = workloads.int4_w()
    xi = workloads.int4_x()
    qi = q.int4g_quantize(dev_bf16(torch, wi))
    rot_i = [tuple(t.clone() for t in qi) for _ in range(8)]
    qa = q.int4g_asym_quantize(dev_bf16(torch, wi))
    rot_a = [tuple(t.clone() for t in qa) for _ in range(8)]
    del qi, qa, wi
    calls = []
    for name, weight, M in DECODE_TRAFFIC:
        if weight == "nvfp4":
            x = dev_bf16(torch, xn[:M])
            a = q.nvfp4_quantize(x)
            y = torch.empty((M, 21504), dtype=torch.bfloat16, device="cuda:0")
            if "w4a4" in name:
                fn = (lambda a, y: lambda i: q.nvfp4_gemm(a, rot_n[i % 16], out=y))(a, y)
            elif "linear" in name:
                fn = (lambda x, a, y: lambda i: q.nvfp4_linear(x, rot_n[i % 16], out=y, x_out=a))(x, a, y)
            else:
                fn = (lambda x, y: lambda i: q.nvfp4_gemm_w4a16(x, rot_n[i % 16], out=y))(x, y)
        else:
            x = dev_bf16(torch, xi[:M])
            y = torch.empty((M, 28672), dtype=torch.bfloat16, device="cuda:0")
            if weight == "int4":
                fn = (lambda x, y: lambda i: q.int4g_gemv(x, *rot_i[i % 8], out=y))(x, y)
            else:
                fn = (lambda x, y: lambda i: q.int4g_asym_gemv(x, *rot_a[i % 8], out=y))(x, y)
        calls.append(fn)
    torch.cuda.synchronize()
    run_copy_calibration(torch)
    k = 0
    for fn in calls:
        for _ in range(launches):
            fn(k)
            k += 1
        torch.cuda.synchronize()
    log(f"decode traffic: {len(calls)} kernels x {launches} launches")
    return {"kernels": [n for n, _, _ in DECODE_TRAFFIC], "launches": launches}


def _counter_rows(path, counter):
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    # one row per dispatch (the value is already summed over the counter's instances)
    by = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        by.setdefault(d, [r["Kernel_Name"], 0.0])
        by[d][1] += float(r["Counter_Value"])
    return [(d, by[d][0], by[d][1]) for d in sorted(by)]


def summarize_decode_traffic(fetch_csv, write_csv, launches=DECODE_TRAFFIC_LAUNCHES):
    """Write DECODE_TRAFFIC_FILE from the counter CSVs of two rocprofv3 --pmc
    runs of `bench.py --decode-traffic` (FETCH_SIZE, then WRITE_SIZE): the
    library's dispatches after the last calibration copy are taken in
    DECODE_TRAFFIC order, `launches` per kernel; counter units become bytes
    with what the same counter reads for the 1 GiB copies; medians per kernel."""
    out_k = {}
    calib = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        copies = [i for i, (_, n, _) in enumerate(rows) if "copyBuffer" in n]
        unit = (1 << 30) / float(np.median([rows[i][2] for i in copies[-3:]]))
        calib[counter] = {"per_GiB_copy": float(np.median([rows[i][2] for i in copies[-3:]])),
                          "bytes_per_unit": unit}
        lib = [(n, v) for (_, n, v) in rows[copies[-1] + 1:] if "nvfp4k::" in n]
        if len(lib) != launches * len(DECODE_TRAFFIC):
            raise ValueError(f"{path}: {len(lib)} library dispatches after the calibration copies, expected "
                             f"{launches * len(DECODE_TRAFFIC)}")
        for j, (name, _, M) in enumerate(DECODE_TRAFFIC):
            chunk = lib[j * launches:(j + 1) * launches]
            kname = {n for n, _ in chunk}
            if len(kname) != 1:
                raise ValueError(f"{name}: mixed kernels {sorted(kname)}")
            e = out_k.setdefault(name, {"kernel": next(iter(kname)).split("(")[0], "M": M,
                                        "algorithmic_bytes": decode_alg_bytes(name, M)})
            e["fetch_bytes" if counter == "FETCH_SIZE" else "write_bytes"] = round(
                float(np.median([v for _, v in chunk])) * unit)
    for e in out_k.values():
        e["traffic_over_algorithmic"] = round((e["fetch_bytes"] + e["write_bytes"]) / e["algorithmic_bytes"], 3)
    cmd = "rocprofv3 --pmc {c} --output-format csv -d <dir> -o {o} -- python3 -u bench.py --decode-traffic"
    out = {
        "workload": "decode-sized calls: NVFP4 weight 21504 x 5376 (16 rotated copies) and INT4 weight 28672 x 8192 "
                    "(group 128, 8 rotated copies), each kernel launched " + str(launches) + " times",
        "kernel_source_hash": kernel_source_hash(DECODE_SOURCES),
        "per_kernel": out_k,
        "calibration": calib,
        "commands": [cmd.format(c="FETCH_SIZE", o="fetch"), cmd.format(c="WRITE_SIZE", o="write"),
                     "python3 bench.py --decode-traffic-from <dir>/fetch_counter_collection.csv "
                     "<dir>/write_counter_collection.csv"],
        "note": "HBM bytes per call = median counter value per dispatch x bytes per counter unit (from the 1 GiB "
                "__amd_rocclr_copyBuffer dispatches of the same run).",
        "hash_note": "sha256 (first 16 hex digits) of " + " + ".join(DECODE_SOURCES) +
                     " with comments and whitespace removed, as bench.py computes it",
    }
    with open(DECODE_TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    return out


def load_decode_traffic():
    """Per-kernel HBM bytes of the decode-sized calls from committed
    counters, or {} if they were taken on different kernel sources."""
    try:
        with open(DECODE_TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("kernel_source_hash") != kernel_source_hash(DECODE_SOURCES):
        return {}
    return t.get("per_kernel", {})


def run_prefill(torch, q, steps, warmup):
    import workloads
    x_bits, wu_bits, wd_bits = workloads.prefill()
    M, N1, K1 = 4096, 21504, 5376
    N2, K2 = 5376, 21504
    x = dev_bf16(torch, x_bits)
    wu = q.nvfp4_quantize(dev_bf16(torch, wu_bits))
    wd = q.nvfp4_quantize(dev_bf16(torch, wd_bits))
    # preallocated buffers: the step allocates nothing
    a1 = (torch.empty((M, K1 // 2), dtype=torch.uint8, device="cuda:0"),
          torch.empty((M, K1 // 16), dtype=torch.uint8, device="cuda:0"),
          torch.empty(1, dtype=torch.float32, device="cuda:0"))
    a2 = (torch.empty((M, K2 // 2), dtype=torch.uint8, device="cuda:0"),
          torch.empty((M, K2 // 16), dtype=torch.uint8, device="cuda:0"),
          torch.empty(1, dtype=torch.float32, device="cuda:0"))
    h = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(q.lib().nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device="cuda:0")
    gws = [torch.empty(max(1, q.lib().nvfp4_gemm_workspace_bytes(M, n, k)), dtype=torch.uint8, device="cuda:0")
           for n, k in ((N1, K1), (N2, K2))]
    del x_bits

    lib = q.lib()
    stream = q._stream(x)
    P = q._ptr

    def quant(inp, a):
        q._check(lib.nvfp4_quantize(P(inp), inp.shape[0], inp.shape[1], P(a[0]), P(a[1]), P(a[2]), 0, P(ws), stream))

    # h's global amax comes from the up GEMM's epilogue (one slot per tile)
    nslots = lib.nvfp4_gemm_amax_slots(M, N1, K1)
    slots = torch.empty(nslots, dtype=torch.int32, device="cuda:0")

    def quant_amax(inp, a):
        q._check(lib.nvfp4_quantize_amax(P(inp), inp.shape[0], inp.shape[1], P(a[0]), P(a[1]), P(a[2]), P(slots),
                                         nslots, stream))

    def gemm_amax(a, w, out, gw):
        q._check(lib.nvfp4_gemm_amax(P(a[0]), P(a[1]), P(a[2]), P(w[0]), P(w[1]), P(w[2]), P(out),
                                     out.shape[0], out.shape[1], a[0].shape[1] * 2, P(gw), gw.numel(), P(slots),
                                     stream))

    def gemm(a, w, out, gw):
        q._check(lib.nvfp4_gemm_ws(P(a[0]), P(a[1]), P(a[2]), P(w[0]), P(w[1]), P(w[2]), P(out),
                                   out.shape[0], out.shape[1], a[0].shape[1] * 2, q.ALGO_TILED, P(gw), gw.numel(),
                                   stream))

    def step():
        quant(x, a1)
        gemm_amax(a1, wu, h, gws[0])
        quant_amax(h, a2)
        gemm(a2, wd, y, gws[1])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps carry no events between their calls: on this GPU every
    # event record between two kernels left the next one idle for ~9 us.
    whole = Timer(torch, stream)
    t = whole.start()
    for i in range(steps):
        step()
        if (i + 1) % max(1, steps // 4) == 0:
            log(f"prefill step {i + 1}/{steps} enqueued")
    whole.stop(t)
    torch.cuda.synchronize()
    ms_step = whole.ms()[0] / steps

    # Per-call durations: `steps` more steps of the same chain with events
    # around each call (the events' gaps fall between the calls; calls
    # repeated back to back would find their weights still in the last-level
    # cache, which the chain evicts).
    timers = [Timer(torch, stream) for _ in range(4)]
    calls = [lambda: quant(x, a1), lambda: gemm_amax(a1, wu, h, gws[0]), lambda: quant_amax(h, a2),
             lambda: gemm(a2, wd, y, gws[1])]
    for _ in range(steps):
        for tm, call in zip(timers, calls):
            t = tm.start()
            call()
            tm.stop(t)
    torch.cuda.synchronize()
    per = [float(np.mean(tm.ms())) for tm in timers]
    quant_ms, gemm_ms = [per[0], per[2]], [per[1], per[3]]
    flops = 2.0 * M * N1 * K1 + 2.0 * M * N2 * K2
    gemm_avg = float(np.mean(gemm_ms))
    return {
        "ms_per_step": ms_step,
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "gemm_avg_ms": gemm_avg,
        "gemm_launches_timed": 2 * steps,
        "gemm_flops_per_launch": 2.0 * M * N1 * K1,
        "gemm_tflops": (2.0 * M * N1 * K1) / (gemm_avg * 1e-3) / 1e12,
        "quant_avg_ms": float(np.mean(quant_ms)),
        "gemm_ms_up_down": gemm_ms,
        "quant_ms_x_h": quant_ms,
    }


def graph_time_us(torch, fn, iters, reps=9):
    """Per-call GPU time of `fn(i)` for i in range(iters), captured once into
    a HIP graph (so host launch overhead does not pace the GPU); the graph is
    replayed `reps` times after two warm-up replays, each replay timed
    between events, and the median replay is reported (clocks and the other
    tenants of the memory system make single replays vary)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) * 1e3 / iters)
    times.sort()
    return times[len(times) // 2]


def run_decode(torch, q, iters=64, copies=16):
    """Decode on the 21504 x 5376 weight at M = 1, 2, 4, 16; GB/s of algorithmic
    bytes.  16 weight copies (~1.04 GB) are rotated so every call misses the
    256 MB last-level cache; calls are replayed from a HIP graph."""
    import workloads
    x_bits, _ = workloads.decode_x()
    w = q.nvfp4_quantize(dev_bf16(torch, workloads.decode_w()))
    ws = [(w[0].clone(), w[1].clone(), w[2].clone()) for _ in range(copies)]
    N, K = 21504, 5376
    out = {}
    for M in (1, 2, 4, 16):
        x = dev_bf16(torch, x_bits[:M])
        a = q.nvfp4_quantize(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        alg_bytes = N * K // 2 + N * K // 16 + 4 + M * K // 2 + M * K // 16 + 4 + M * N * 2
        ref = q.nvfp4_gemm(a, ws[(iters - 1) % copies]).clone()
        us = graph_time_us(torch, lambda i: q.nvfp4_gemm(a, ws[i % copies], out=y), iters)
        assert torch.equal(y, ref), "graph replay differs from the eager call"

        # nvfp4_linear: one kernel at M <= 2 (the GEMV quantizes x itself),
        # quantize + GEMM above
        nbytes = q.lib().nvfp4_linear_workspace_bytes(M, N, K)
        lws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0") if nbytes else None
        us_q = graph_time_us(torch, lambda i: q.nvfp4_linear(x, ws[i % copies], out=y, x_out=a, workspace=lws),
                             iters)
        assert torch.equal(y, ref), "nvfp4_linear differs from quantize + gemm"
        out[f"M{M}"] = {"us": us, "GBps": alg_bytes / (us * 1e-6) / 1e9,
                        "frac_hbm": alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "us_incl_act_quant": us_q, "alg_bytes": alg_bytes}
        log(f"decode M={M}: {us:.2f} us, {out[f'M{M}']['GBps']:.0f} GB/s; incl. act quant {us_q:.2f} us")
    # weight-only mode: bf16 activation straight into the GEMV (no quantization)
    for M in (1, 2, 4, 16):
        x = dev_bf16(torch, x_bits[:M])
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        alg_bytes = N * K // 2 + N * K // 16 + 4 + M * K * 2 + M * N * 2
        ref = q.nvfp4_gemm_w4a16(x, ws[(iters - 1) % copies]).clone()
        us = graph_time_us(torch, lambda i: q.nvfp4_gemm_w4a16(x, ws[i % copies], out=y), iters)
        assert torch.equal(y, ref), "graph replay differs from the eager call"
        out[f"w4a16_M{M}"] = {"us": us, "GBps": alg_bytes / (us * 1e-6) / 1e9,
                              "frac_hbm": alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "alg_bytes": alg_bytes}
        log(f"decode W4A16 M={M}: {us:.2f} us, {out[f'w4a16_M{M}']['GBps']:.0f} GB/s")
    # weight-only past decode sizes: the prefill activation through the MFMA tiles
    Mp = 4096
    x = dev_bf16(torch, workloads.normal_bf16("prefill", 0, (4096, 5376)))   # the prefill x_up
    y = torch.empty((Mp, N), dtype=torch.bfloat16, device="cuda:0")
    ms = min(_event_ms(torch, lambda: q.nvfp4_gemm_w4a16(x, ws[0], out=y), 3) for _ in range(3))
    out[f"w4a16_M{Mp}"] = {"ms": ms, "tflops": 2 * Mp * N * K / (ms * 1e-3) / 1e12}
    log(f"W4A16 M={Mp} (tiled): {ms:.3f} ms, {out[f'w4a16_M{Mp}']['tflops']:.0f} TFLOP/s")
    del ws, x, y
    # HBM bytes per call from committed rocprofv3 counters (None once the
    # kernels have changed since they were taken)
    tr = load_decode_traffic()
    for key, name in [(f"M{m}", f"nvfp4_w4a4_M{m}") for m in (1, 2, 4, 16)] + \
                     [(f"w4a16_M{m}", f"nvfp4_w4a16_M{m}") for m in (1, 2, 4, 16)]:
        t = tr.get(name)
        out[key]["traffic_bytes"] = t["fetch_bytes"] + t["write_bytes"] if t else None
    for m in (1, 2):
        t = tr.get(f"nvfp4_linear_M{m}")
        out[f"M{m}"]["traffic_bytes_incl_act_quant"] = t["fetch_bytes"] + t["write_bytes"] if t else None
    return out


def run_weight_quant(torch, q, reps=5):
    """Offline weight quantization of W_up [21504, 5376] under each block-scale
    rule (absmax, four-over-six, MSE): time per call and GB/s of algorithmic
    bytes (2 B read + 0.5625 B written per element)."""
    import workloads
    w = dev_bf16(torch, workloads.decode_w())
    n = w.numel()
    out = {}
    for rule in ("absmax", "four_over_six", "mse"):
        q.nvfp4_quantize(w, rule=rule)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            q.nvfp4_quantize(w, rule=rule)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        out[rule] = {"us": us, "GBps": n * 2.5625 / (us * 1e-6) / 1e9}
        log(f"weight quant {rule}: {us:.1f} us, {out[rule]['GBps']:.0f} GB/s")
    return out


def run_dit(torch, q, reps=3):
    """4 denoising steps x (qkv, up, down) with fresh activations; TFLOP/s incl. act quant
    (the up projection's output is quantized from the amax its GEMM leaves)."""
    import workloads
    wq, wu, wd = [q.nvfp4_quantize(dev_bf16(torch, b)) for b in workloads.dit_weights()]
    xs = [dev_bf16(torch, workloads.dit_x(t)) for t in range(4)]
    flops = 4 * 2.0 * 4096 * 3072 * (9216 + 12288 + 12288)

    def run():
        for t in range(4):
            a = q.nvfp4_quantize(xs[t])
            q.nvfp4_gemm(a, wq)
            hh, slots = q.nvfp4_gemm_amax(a, wu)
            q.nvfp4_gemm(q.nvfp4_quantize_amax(hh, slots), wd)

    run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    log(f"dit 4 steps: {ms:.3f} ms")
    return {"ms_4_steps": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def _event_ms(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def run_lora(torch, q, reps=10, rank=32):
    """Run-time low-rank branch next to the NVFP4 product: the diffusion qkv
    layer [4096 x 3072] x [9216 x 3072] with a rank-32 adapter (quantize with
    the fused down projection, then the GEMM with the branch in its epilogue)
    against the same layer without it; and decode M=1 on the 21504 x 5376
    weight with a rank-32 adapter."""
    import workloads
    x = dev_bf16(torch, workloads.dit_x(0))
    w = q.nvfp4_quantize(dev_bf16(torch, workloads.dit_weights()[0]))
    down, up = [dev_bf16(torch, b) for b in workloads.dit_lora(rank)]
    M, N, K = 4096, 9216, 3072
    a = q.nvfp4_quantize(x)
    t = torch.empty((M, rank), dtype=torch.float32, device="cuda:0")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    g = torch.empty(1, dtype=torch.float32, device="cuda:0")
    a_l = (torch.empty_like(a[0]), torch.empty_like(a[1]), g)

    def plain():
        q.nvfp4_quantize(x, out=a)
        q.nvfp4_gemm(a, w, out=y)

    def lora():
        q.nvfp4_quantize_lora(x, down, out=(a_l[0], a_l[1], g, t))
        q.nvfp4_gemm_lora(a_l, w, t, up, out=y)

    out = {"rank": rank}
    out["dit_qkv_ms"] = _event_ms(torch, plain, reps)
    out["dit_qkv_lora_ms"] = _event_ms(torch, lora, reps)
    out["dit_qkv_quant_ms"] = _event_ms(torch, lambda: q.nvfp4_quantize(x, out=a), reps)
    out["dit_qkv_quant_lora_ms"] = _event_ms(torch, lambda: q.nvfp4_quantize_lora(x, down, out=(a_l[0], a_l[1], g, t)),
                                             reps)
    out["dit_qkv_gemm_ms"] = _event_ms(torch, lambda: q.nvfp4_gemm(a, w, out=y), reps)
    out["dit_qkv_gemm_lora_ms"] = _event_ms(torch, lambda: q.nvfp4_gemm_lora(a_l, w, t, up, out=y), reps)
    flops = 2.0 * M * N * K
    out["dit_qkv_tflops"] = flops / (out["dit_qkv_ms"] * 1e-3) / 1e12
    out["overhead_frac"] = out["dit_qkv_lora_ms"] / out["dit_qkv_ms"] - 1.0
    log(f"lora r={rank} dit qkv: {out['dit_qkv_ms']:.3f} ms plain, {out['dit_qkv_lora_ms']:.3f} ms with the branch "
        f"(quant {out['dit_qkv_quant_ms']:.3f} -> {out['dit_qkv_quant_lora_ms']:.3f}, "
        f"gemm {out['dit_qkv_gemm_ms']:.3f} -> {out['dit_qkv_gemm_lora_ms']:.3f})")
    # decode M = 1 with the branch (weights rotated past the last-level cache)
    xd, _ = workloads.decode_x()
    wd = q.nvfp4_quantize(dev_bf16(torch, workloads.decode_w()))
    copies, iters = 16, 64
    ws = [(wd[0].clone(), wd[1].clone(), wd[2].clone()) for _ in range(copies)]
    Nd, Kd = 21504, 5376
    x1 = dev_bf16(torch, xd[:1])
    dn1 = dev_bf16(torch, workloads.random_bf16(77, (rank, Kd), sigma=0.02))
    up1 = dev_bf16(torch, workloads.random_bf16(78, (Nd, rank), sigma=0.02))
    a1 = q.nvfp4_quantize(x1)
    t1 = torch.empty((1, rank), dtype=torch.float32, device="cuda:0")
    y1 = torch.empty((1, Nd), dtype=torch.bfloat16, device="cuda:0")
    out["decode_m1_us"] = graph_time_us(torch, lambda i: q.nvfp4_gemm(a1, ws[i % copies], out=y1), iters)
    out["decode_m1_lora_us"] = graph_time_us(torch, lambda i: q.nvfp4_gemm_lora(a1, ws[i % copies], t1, up1, out=y1),
                                             iters)

    def dec_full(i):
        q.nvfp4_quantize_lora(x1, dn1, out=(a1[0], a1[1], a1[2], t1))
        q.nvfp4_gemm_lora(a1, ws[i % copies], t1, up1, out=y1)
    out["decode_m1_lora_incl_quant_us"] = graph_time_us(torch, dec_full, iters)
    log(f"lora r={rank} decode M=1: {out['decode_m1_us']:.2f} us plain, {out['decode_m1_lora_us']:.2f} us with the "
        f"branch, {out['decode_m1_lora_incl_quant_us']:.2f} us incl. quantize + down projection")
    del ws
    return out


def run_int4(torch, q, iters=64, copies=8):
    import workloads
    w_bits = workloads.int4_w()
    x_bits = workloads.int4_x()
    N, K = 28672, 8192
    qq, ss = q.int4g_quantize(dev_bf16(torch, w_bits))
    del w_bits
    rot = [(qq.clone(), ss.clone()) for _ in range(copies)]      # ~0.97 GB rotated
    out = {}
    tr = load_decode_traffic()
    for M in (1, 4, 16):
        x = dev_bf16(torch, x_bits[:M])
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        alg_bytes = N * K // 2 + N * (K // 128) * 2 + M * K * 2 + M * N * 2
        ref = q.int4g_gemv(x, *rot[(iters - 1) % copies]).clone()
        us = graph_time_us(torch, lambda i: q.int4g_gemv(x, *rot[i % copies], out=y), iters)
        assert torch.equal(y, ref), "graph replay differs from the eager call"
        t = tr.get(f"int4_M{M}")
        out[f"M{M}"] = {"us": us, "GBps": alg_bytes / (us * 1e-6) / 1e9,
                        "frac_hbm": alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "traffic_bytes": t["fetch_bytes"] + t["write_bytes"] if t else None}
        log(f"int4 M={M}: {us:.2f} us, {out[f'M{M}']['GBps']:.0f} GB/s")
    x = dev_bf16(torch, x_bits)
    y = torch.empty((2048, N), dtype=torch.bfloat16, device="cuda:0")
    q.int4g_gemv(x, qq, ss, out=y)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(5):
        q.int4g_gemv(x, qq, ss, out=y)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / 5
    out["M2048"] = {"ms": ms, "tflops": 2.0 * 2048 * N * K / (ms * 1e-3) / 1e12}
    log(f"int4 M=2048: {ms:.3f} ms")
    del rot
    # asymmetric (zero-point) variant of the same weight, M = 1
    import workloads
    qa, sa, za = q.int4g_asym_quantize(dev_bf16(torch, workloads.int4_w()))
    rot = [(qa.clone(), sa.clone(), za.clone()) for _ in range(copies)]
    del qa, sa, za
    x = dev_bf16(torch, x_bits[:1])
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda:0")
    alg_bytes = N * K // 2 + N * (K // 128) * 3 + K * 2 + N * 2
    ref = q.int4g_asym_gemv(x, *rot[(iters - 1) % copies]).clone()
    us = graph_time_us(torch, lambda i: q.int4g_asym_gemv(x, *rot[i % copies], out=y), iters)
    assert torch.equal(y, ref), "graph replay differs from the eager call"
    t = tr.get("int4_asym_M1")
    out["asym_M1"] = {"us": us, "GBps": alg_bytes / (us * 1e-6) / 1e9,
                      "frac_hbm": alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                      "traffic_bytes": t["fetch_bytes"] + t["write_bytes"] if t else None}
    log(f"int4 asym M=1: {us:.2f} us, {out['asym_M1']['GBps']:.0f} GB/s")
    # M = 2048 on the tile kernel (group sums of x on the matrix cores)
    xa = dev_bf16(torch, x_bits)
    ya = torch.empty((2048, N), dtype=torch.bfloat16, device="cuda:0")
    ms = _event_ms(torch, lambda: q.int4g_asym_gemv(xa, *rot[0], out=ya), 5)
    out["asym_M2048"] = {"ms": ms, "tflops": 2.0 * 2048 * N * K / (ms * 1e-3) / 1e12}
    log(f"int4 asym M=2048: {ms:.3f} ms")
    del rot
    return out



PEAK_LIB = os.path.join(ROOT, "peak", "libpeak.so")


def run_peaks(torch, iters=64, copies=16):
    """Measured roofline denominators (peak/peak.hip): the dense fp16 MFMA
    issue loop over the whole chip (TFLOP/s), the tiled GEMM's 32x32x16 MFMA
    with operand data of three kinds and with vector instructions between
    the MFMAs, a 1 GiB non-temporal read
    (GB/s), and the per-call time of a plain read of the decode weight's
    bytes (65,074,136) over 16 rotated buffers, replayed from a HIP graph as
    the decode calls are (the floor a decode call could reach)."""
    import ctypes
    if not os.path.exists(PEAK_LIB):
        raise RuntimeError(f"{PEAK_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(PEAK_LIB)
    lib.peak_out_elems.restype = ctypes.c_int
    lib.peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.peak_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    out = torch.empty(lib.peak_out_elems(), dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def check(err, what):
        if err != 0:
            raise RuntimeError(f"{what}: HIP error {err}")

    flops = ctypes.c_double()
    for _ in range(3):
        check(lib.peak_mfma(4096, ctypes.c_void_p(out.data_ptr()), ctypes.byref(flops), stream), "peak_mfma")
    reps = 10
    ms = _event_ms(torch, lambda: [check(lib.peak_mfma(4096, ctypes.c_void_p(out.data_ptr()), ctypes.byref(flops),
                                                       stream), "peak_mfma") for _ in range(reps)], 1) / reps
    mfma = flops.value / (ms * 1e-3) / 1e12
    # the tiled GEMM's v_mfma_f32_32x32x16_f16 at one wave per SIMD, operands
    # changing every instruction: zeros / E2M1 x E4M3 products / random fp16,
    # and with 2 or 4 vector instructions after every MFMA (products data)
    # ("_hold": the first operand held for eight MFMAs, the GEMM's order)
    lib.peak_mfma_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    mix = {}
    for mode, valu, hold in ((0, 0, 0), (1, 0, 0), (2, 0, 0), (1, 2, 0), (1, 4, 0), (1, 0, 1), (1, 2, 1)):
        def run_mix(mode=mode, valu=valu, hold=hold):
            check(lib.peak_mfma_mix(16384, mode, valu, hold, ctypes.c_void_p(out.data_ptr()), ctypes.byref(flops),
                                    stream), "peak_mfma_mix")
        for _ in range(2):
            run_mix()
        ms_m = _event_ms(torch, lambda: [run_mix() for _ in range(5)], 1) / 5
        name = ("zeros", "e2m1_x_e4m3", "random_f16")[mode]
        mix[f"{name}_valu{valu}" + ("_hold" if hold else "")] = flops.value / (ms_m * 1e-3) / 1e12
    # reads: the best of three grid sizes (2, 4, 8 workgroups per CU)
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    big.fill_(1)
    read, read_wgs = 0.0, 0
    for wgs in (2, 4, 8):
        ms_r = _event_ms(torch, lambda: [check(lib.peak_read(ctypes.c_void_p(big.data_ptr()), big.numel(), wgs,
                                                             ctypes.c_void_p(out.data_ptr()), stream), "peak_read")
                                         for _ in range(reps)], 1) / reps
        if big.numel() / (ms_r * 1e-3) / 1e9 > read:
            read, read_wgs = big.numel() / (ms_r * 1e-3) / 1e9, wgs
    # the same stream through LDS by DMA (how the GEMM kernels copy operands)
    ms_l = _event_ms(torch, lambda: [check(lib.peak_read_lds(ctypes.c_void_p(big.data_ptr()), big.numel(),
                                                             ctypes.c_void_p(out.data_ptr()), stream), "peak_read_lds")
                                     for _ in range(reps)], 1) / reps
    read_lds = big.numel() / (ms_l * 1e-3) / 1e9
    del big
    nb = 65074136
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    floor_us, floor_wgs = float("inf"), 0
    for wgs in (2, 4, 8):
        def one(i, wgs=wgs):
            s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            check(lib.peak_read(ctypes.c_void_p(bufs[i % copies].data_ptr()), nb, wgs, ctypes.c_void_p(out.data_ptr()),
                                s), "peak_read")
        us = graph_time_us(torch, one, iters)
        if us < floor_us:
            floor_us, floor_wgs = us, wgs
    del bufs
    res = {"mfma_f16_tflops": mfma, "mfma_frac_of_spec": mfma / PEAK_MFMA_TFLOPS,
           "hbm_read_gbs": read, "hbm_frac_of_spec": read / PEAK_HBM_GBS, "read_wgs_per_cu": read_wgs,
           "hbm_read_lds_dma_gbs": read_lds,
           "decode_read_floor_us": floor_us, "decode_read_floor_gbs": nb / (floor_us * 1e-6) / 1e9,
           "floor_wgs_per_cu": floor_wgs,
           "mfma_32x32x16_f16_one_wave_per_simd_tflops": mix}
    log(f"peaks: MFMA fp16 loop {mfma:.0f} TFLOP/s ({mfma / PEAK_MFMA_TFLOPS:.3f} of spec), 1 GiB read "
        f"{read:.0f} GB/s ({read_lds:.0f} GB/s through LDS by DMA), 65 MB read per call (graph) {floor_us:.2f} us")
    log("peaks: 32x32x16 MFMA loop, one wave per SIMD (TFLOP/s): " +
        ", ".join(f"{k} {v:.0f}" for k, v in mix.items()))
    return res


def run_copy_calibration(torch, nbytes=1 << 30):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {nbytes} bytes")


def cpu_baseline(rows=256):
    """The CPU oracle as it stands, timed on the host on bounded samples of
    the configurations (tens of seconds in all):
    - value: the prefill up projection, `rows` of its 4096 activation rows
      (quantized with the whole tensor's g, as the method defines it), then
      the fp64 GEMM of those rows against W_up, in TFLOP/s (the headline's
      unit), BLAS on all cores;
    - quantizer: the oracle's NVFP4 quantizer on one core (BLAS limited to
      one thread) on activation and weight row samples, GB/s at 2.5625 B per
      element (2 read, 0.5 + 1/16 written);
    - per_config: the oracle's fp64 GEMM (weight decode included) in GFLOP/s
      for each configuration, on the sample each entry names;
    - the host: CPU model, cores this process may use, and the BLAS
      libraries with their thread counts (threadpoolctl)."""
    import threadpoolctl
    import workloads
    from oracle import intq as I
    from oracle import nvfp4 as O
    info = threadpoolctl.threadpool_info()
    blas = [{k: i.get(k) for k in ("user_api", "internal_api", "version", "num_threads", "threading_layer")}
            for i in info]
    threads = max([i.get("num_threads", 1) for i in info] or [1])

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    x_bits, wu_bits, _ = workloads.prefill()
    wq = O.quantize(wu_bits)                      # offline weight quantization, not timed
    sample = np.asarray(x_bits[:rows])
    g = O.global_scale(x_bits)
    a, dt_q = timed(lambda: O.quantize(sample, g=g))
    _, dt_g = timed(lambda: O.gemm(*a, *wq))
    dt = dt_q + dt_g
    flops = 2.0 * rows * 21504 * 5376
    per = {}
    per["prefill_up"] = {"gflops": flops / dt_g / 1e9, "seconds": dt_g,
                         "sample": f"{rows} x 5376 activation rows x W_up [21504, 5376]"}
    # quantizer on one core
    with threadpoolctl.threadpool_limits(1):
        _, dq_x = timed(lambda: O.quantize(sample, g=g))
        wsample = np.asarray(wu_bits[:2048])
        _, dq_w = timed(lambda: O.quantize(wsample))
    quant = {"activation_gbs": sample.size * 2.5625 / dq_x / 1e9, "activation_sample": f"{rows} x 5376 of x_up",
             "weight_gbs": wsample.size * 2.5625 / dq_w / 1e9, "weight_sample": "2048 x 5376 of W_up",
             "threads": 1}
    # fp64 GEMM per configuration (BLAS on all cores)
    ta, tw = workloads.tiny()
    oa, ow = O.quantize(ta), O.quantize(tw)
    _, d = timed(lambda: O.gemm(*oa, *ow))
    per["tiny"] = {"gflops": 2.0 * 16 * 256 * 256 / d / 1e9, "seconds": d, "sample": "whole: 16 x 256 x 256"}
    xd, _ = workloads.decode_x()
    ad = O.quantize(xd[:16])
    _, d = timed(lambda: O.gemm(*ad, *wq))
    per["decode_M16"] = {"gflops": 2.0 * 16 * 21504 * 5376 / d / 1e9, "seconds": d,
                         "sample": "whole: M = 16 x W [21504, 5376]"}
    del wq, wu_bits, x_bits
    wqkv = workloads.dit_weights()[0][:1024]
    xq = workloads.dit_x(0)
    aq = O.quantize(xq[:256], g=O.global_scale(xq))
    wqq = O.quantize(wqkv)
    _, d = timed(lambda: O.gemm(*aq, *wqq))
    per["dit_qkv"] = {"gflops": 2.0 * 256 * 1024 * 3072 / d / 1e9, "seconds": d,
                      "sample": "256 of 4096 activation rows x 1024 of 9216 qkv weight rows, K = 3072"}
    w4 = workloads.int4_w()[:4096]
    x4 = workloads.int4_x()[:16]
    p4, s4, _ = I.int4g_quantize(w4)
    _, d = timed(lambda: I.int4g_gemm(x4, p4, s4))
    per["int4_M16"] = {"gflops": 2.0 * 16 * 4096 * 8192 / d / 1e9, "seconds": d,
                       "sample": "M = 16 x 4096 of 28672 weight rows, K = 8192"}
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of 4096 rows of the prefill up projection (quantize + fp64 GEMM incl. weight decode), "
                      f"{dt:.1f} s", "seconds": dt,
            "quantizer_1core": quant, "per_config": per, "blas": blas,
            "cpu": _cpu_model(), "host_cores": len(os.sched_getaffinity(0))}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="only the prefill step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["decode", "dit", "int4", "weight_quant", "lora", "peaks"],
                    help="time only this extra workload")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the GEMM traffic summary from two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--decode-traffic", action="store_true",
                    help="launch each decode-sized kernel a few times for rocprofv3 --pmc and exit")
    ap.add_argument("--decode-traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the decode traffic summary from two rocprofv3 --pmc runs and exit (no GPU)")
    args = ap.parse_args()
    if args.traffic_from:
        out = summarize_traffic(*args.traffic_from)
        print(json.dumps({"traffic_bytes_per_launch": out["bytes_per_launch"], "file": TRAFFIC_FILE}))
        return
    if args.decode_traffic_from:
        out = summarize_decode_traffic(*args.decode_traffic_from)
        print(json.dumps({k: v["traffic_over_algorithmic"] for k, v in out["per_kernel"].items()}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path runs on a "
              f"single GPU; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_gemm_nvfp4_amd as q
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q.lib()
    log(f"device {torch.cuda.get_device_name(0)}")

    if args.decode_traffic:
        print(json.dumps(run_decode_traffic(torch, q)))
        return
    if args.only:
        res = {"decode": run_decode, "dit": run_dit, "int4": run_int4, "weight_quant": run_weight_quant,
               "lora": run_lora, "peaks": lambda t, _: run_peaks(t)}[args.only](torch, q)
        print(json.dumps({"only": args.only, "result": res}))
        return
    peaks = run_peaks(torch)
    pre = run_prefill(torch, q, args.steps, args.warmup)
    log(f"prefill: {pre['ms_per_step']:.3f} ms/step, {pre['tflops']:.1f} TFLOP/s incl. act quant; "
        f"tiled GEMM {pre['gemm_avg_ms']:.3f} ms ({pre['gemm_tflops']:.1f} TFLOP/s)")
    extras = {}
    if not args.no_extras:
        extras["decode"] = run_decode(torch, q)
        extras["dit"] = run_dit(torch, q)
        extras["int4"] = run_int4(torch, q)
        extras["weight_quant"] = run_weight_quant(torch, q)
        extras["lora"] = run_lora(torch, q)
    if args.copy_calibration:
        run_copy_calibration(torch)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads; quantizer 1 core "
            f"{cpu['quantizer_1core']['activation_gbs']:.3f} GB/s; "
            + ", ".join(f"{k} {v['gflops']:.1f} GFLOP/s" for k, v in cpu["per_config"].items()))

    achieved = pre["gemm_tflops"]
    line = {
        "metric": METRIC,
        "value": round(pre["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "prefill MLP M=4096: quantize x[4096,5376] + NVFP4 GEMM vs W_up[21504,5376] "
                               "(with h's amax), quantize h[4096,21504] + NVFP4 GEMM vs W_down[5376,21504]",
                   "M": 4096, "N_up": 21504, "K_up": 5376, "N_down": 5376, "K_down": 21504,
                   "format": "E2M1 codes, E4M3 scale per 16, fp32 per-tensor scale"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": load_traffic(),
                     "kernel": "nvfp4_gemm_tiled_kernel (+ nvfp4_gemm_tiled_reduce_kernel: one GEMM call)",
                     "avg_launch_ms": round(pre["gemm_avg_ms"], 4),
                     "peak_measured": round(peaks["mfma_f16_tflops"], 1),
                     "frac_measured": round(achieved / peaks["mfma_f16_tflops"], 4),
                     # the same instruction on the operand values the GEMM feeds it (decoded
                     # E2M1 x E4M3 products) with 2 vector instructions per MFMA, as in its loop
                     "peak_measured_products": round(peaks["mfma_32x32x16_f16_one_wave_per_simd_tflops"]
                                                     ["e2m1_x_e4m3_valu2_hold"], 1),
                     "frac_measured_products": round(achieved / peaks["mfma_32x32x16_f16_one_wave_per_simd_tflops"]
                                                     ["e2m1_x_e4m3_valu2_hold"], 4)},
        "peaks": {k: (round(v, 4) if isinstance(v, float) else
                      ({kk: round(vv, 1) for kk, vv in v.items()} if isinstance(v, dict) else v))
                  for k, v in peaks.items()},
        "cpu_baseline": cpu,
        "prefill": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in pre.items()},
    }
    if extras:
        d1 = extras["decode"]["M1"]
        line["decode_m1"] = {"value": round(d1["GBps"], 1), "unit": "GB/s", "frac_hbm": round(d1["frac_hbm"], 4),
                             "us": round(d1["us"], 2), "us_incl_act_quant": round(d1["us_incl_act_quant"], 2),
                             "alg_bytes": d1["alg_bytes"], "traffic": d1.get("traffic_bytes"),
                             "kernel": "nvfp4_gemv_stream_kernel<1, 3, false>",
                             "frac_hbm_measured": round(d1["GBps"] / peaks["hbm_read_gbs"], 4),
                             "read_floor_us": round(peaks["decode_read_floor_us"], 2)}
        line["extras"] = extras
    print(json.dumps(line))


if __name__ == "__main__":
    main()
