"""Double-precision CPU oracle for the single-GPU MoE-layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or constants with the HIP path under ``mixture_experts_layer_04_amd``
and it imports nothing from there.

It is deliberately plain and slow: every floating-point step is carried out in
float64 on exactly widened stored values (bf16 bits, fp32 gate and bias, OCP
fp8 / fp4 codes with their scales), in the order the pages describe.

Sources (web pages; cited by title and section throughout):

* [Router] "How an MoE Model Picks Its Experts During LLM Inference"
  (vincentzed.com/writing/moe-router-gemm)
* [MoE] "Mixture of Experts" (mlinterviewnotes.com, inference course,
  chapter 07-01)
* [Kernels] "MoE Kernels, in depth: the six kernels of an expert layer ..."
  (aicassindra.com/blogs/gpu/gpu_moe_kernels.html)
* [MegaMoE] "How GPUs Fuse Communication and Computation During LLM
  Inference" (vincentzed.com/writing/megamoe)

Modules:

* ``formats`` - exact decoders for bf16, OCP E4M3FN, E2M1 and E8M0 and the
  round-to-nearest-even e4m3 quantiser used by the emulate mode.
* ``router``  - gate logits, scoring, rank keys, group limit, k-round top-k,
  weights and the cut / group margins.
* ``align``   - block alignment (histogram, padding, scan, stable placement,
  block table, padded length).
* ``ffn``     - expert weights dequantised exactly, SwiGLU expert, activation
  quantisation (emulate mode), direct and grouped combine, full layer.

Parity status of each function is stated in its docstring ("pinned by ..."
or "parity unpinned").
"""

from . import formats, router, align, ffn  # noqa: F401
