"""CPU oracle for NVFP4 block quantization, the block-scaled 4-bit GEMM, and
the symmetric per-group integer (INT4/INT8) weight-only scheme.

This package is TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP kernels behind ``include/nvfp4.h`` and
the Python binding ``quantized_gemm_nvfp4_amd``) never imports, links or calls
anything here, and nothing here imports the product path: the two share no
code, tables or constants.

Everything is plain numpy, written from the pages' definitions:

* ``formats``  -- the element and scale number formats: E2M1 (4-bit float),
  FP8 E4M3 ("float8_e4m3fn"), and the bf16 / fp16 round-to-nearest-even casts.
* ``nvfp4``    -- NVFP4 quantize / dequantize and the block-scaled GEMM.
* ``scale_rules`` -- block-scale selection: absmax, four-over-six, MSE.
* ``lora``     -- the run-time low-rank branch next to the NVFP4 product.
* ``intq``     -- the symmetric integer formula and its INT4 per-group form.
* ``metrics``  -- the parity metrics (relative L2, per-row max-abs).

Parity status of every function is stated in its module header.  All
functions are pinned by the CPU tests in ``tests/test_oracle_*.py`` (worked
examples, closed forms, brute force on tiny inputs, library casts).
"""
