"""Plain, slow, fp64 CPU oracle for the sparse-MoE expert-decode path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls, links or imports anything here, and
nothing here imports the HIP library or its Python binding: the two sides
share no code.  Inputs for both come from the seeded generators in ``synth``,
which hold none of the method's arithmetic.

Every function restates a plain definition in NumPy float64:

* ``formats``  - MXFP4 (E2M1 codes + E8M0 block scales) and group-quantized
  int4 decoding; the dequantized fp32 weights are exact results.
* ``gemv``     - y = W.x in fp64 plus the normaliser sum |W||x|.
* ``moe``      - RMSNorm, router logits, top-k with softmax weights, the
  SiLU-gated SwiGLU expert FFN, the router-weighted combine, and the
  residual layer stack (layer-major evaluation, optional teacher forcing).
* ``mxq``      - MXFP8 (E4M3 + E8M0 per 32) quantization of activations and
  the MX-scaled product of MXFP4 weights with MXFP8 activations (the
  large-M / prefill GEMM).
* ``attn``     - decode attention of a gpt-oss layer: YaRN inverse
  frequencies and attention scaling, the rotary table and the rotation that
  feeds the KV cache, and causal attention with learned per-head sinks over a
  full or sliding window.

Where the pages leave a step open (they print no formula: the Methods
sections of all three octopusresearch pages are empty) each module states the
reading it takes.
"""

from . import attn, formats, gemv, moe, mxq  # noqa: F401
