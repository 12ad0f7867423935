"""CPU oracle for the routed mixture-of-experts layer — TEST INFRASTRUCTURE.

A plain, slow, obviously correct float64 implementation of what the layer
computes, written from the definitions and sharing no code with the GPU
library (no kernels, headers, tables or helpers in common).  Only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it; the product path never does.

What the layer computes, and where each part comes from:

* weights are read in their checkpoint format with no dequantized copy
  ("DGPP" README, intro bullet on serving checkpoints as published; forum
  thread "DGPP: a GB10-optimized C++/CUDA inference engine", opening post,
  quantization table: NVFP4 / MXFP4 routed experts, FP8 block-128 shared
  experts, activations BF16);
* element and scale encodings follow the public OCP specifications (OCP
  Microscaling Formats v1.0 for E2M1 and E8M0; OCP 8-bit Floating Point for
  E4M3), the NVFP4 layout (E2M1 x E4M3 per 16 x fp32 tensor scale) as the
  checkpoint format the pages serve;
* per-expert partial sums are combined in fp32 by default, bf16 partials
  being an explicit lossy lever (gitee "dgpp" README, "Execution and
  performance" table, key ``engine.prefill_bf16_partials``);
* activations stay BF16: the W4A4 path is opt-in and calibration scales no
  longer enable activation quantization (forum thread, page 5, the update
  post on NVFP4 W4A4 prefill).

The router function (softmax, top-k, renormalisation), SwiGLU, the shared
expert and tie rules are not on the pages; the readings taken are listed in
the module docstring of :mod:`oracle.layer`.

Submodules: :mod:`oracle.formats` (decoders), :mod:`oracle.layer` (the layer),
:mod:`oracle.lossy` (the opt-in activation-quantizing modes, mirrored).
"""
from . import formats, layer, lossy  # noqa: F401
