"""CPU oracle for the W8A8 / block-scaled FP8 / SmoothQuant INT8 / MXFP4 / NVFP4 / W4A16 hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library (``fp4_w8a8_quantized_amd``)
and never imports it; the only module both sides use is ``synthetic`` (seeded input
generators, which hold none of the method's arithmetic).

Everything here is plain NumPy on the CPU, written from the definitions on three pages:

* [P-FP8FP4]  "FP8 and FP4 inference, SmoothQuant and activation quantization"
* [P-FP8INT8] "FP8 and INT8 Inference"
* [P-LOWBIT]  "Low-bit LLM Weights and Activations"

Each function names the section it follows. Floating-point work is done in fp64 unless
the pages fix the precision: the scale and quotient arithmetic of the quantizers runs in
IEEE fp32, because the pages' emulation of per-token quantization runs on fp32 tensors
and an integer (the code) is decided by it.

Pinning status (what each part is checked against lives in ``tests/test_oracle_*.py``):

* formats.py      pinned (page values, exhaustive brute force, torch CPU casts)
* quant.py        pinned (worked example printed on [P-FP8INT8] §4, brute force, invariants)
* gemm.py         pinned (brute force, scale-factoring identity, [P-FP8FP4] worked example)
* smoothquant.py  pinned (closed forms printed on [P-LOWBIT] Try-it 02 and [P-FP8FP4])
* roofline.py     pinned (numbers printed on [P-FP8FP4] and [P-LOWBIT] §5)
* epilogue.py     pinned (options off = the plain references; SiLU closed forms and an
                  independent routine; hand-computed INT8 order and FP8-code examples)
* static_scale.py pinned (one row at its own amax scale = the dynamic quantizer; hand
                  saturation counts; a worked delayed-scaling window)
* nvfp4.py        pinned (hand-computed grid blocks and scale codes, nearest-value brute
                  force, the zero-scale rule, 4.5 bits per element from [P-LOWBIT] §2.4,
                  triple-loop GEMM)
* w4a16.py        pinned (metadata sizes printed on [P-LOWBIT] §2.3 / §3.3, a hand-computed
                  group, nearest-integer brute force, packing, triple-loop GEMM)
"""

from . import formats, quant, gemm, smoothquant, roofline, epilogue, static_scale, nvfp4, w4a16  # noqa: F401

__all__ = ["formats", "quant", "gemm", "smoothquant", "roofline", "epilogue", "static_scale", "nvfp4", "w4a16"]
