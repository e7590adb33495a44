"""CPU oracle for the fused scaled linear: plain, slow, fp64, obviously correct.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, tables or
helpers with ``scaled_gemm_epilogues_amd`` (the HIP path), and it never reads
a value the HIP path produced.

Sources (web pages, cited by title and section):

* "NVIDIA TransformerEngine Ops Fused Forward Linear Scale Add" (leeroopedia),
  Description and I/O Contract: ``output = residual + scale * (input @ weight^T)``
  written into the residual buffer.
* "NVIDIA TransformerEngine Ops Fused Backward Linear Scale" (leeroopedia),
  Description and I/O Contract: the scale is passed as the alpha of both the
  dgrad and the wgrad GEMM ("scaled dgrad", "scaled weight gradient").
* "NVIDIA TransformerEngine PyTorch Ext Normalization" (leeroopedia),
  Description: FP8 current scaling is "amax, then quantize"; MXFP8 is a
  quantized output format.
* "core.tensor_parallel.inference_layers" (Megatron-core API docs),
  ``_apply_linear``: the GEMM is chosen by operand type (MXFP8 or standard).
* "Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
  (TransformerEngine PR 3238): scaled SwiGLU, grouped linear, precomputed
  split offsets (Description; Greptile Summary; Sequence Diagram).
* "NVIDIA TransformerEngine PyTorch Ext Normalization" (leeroopedia), Description and I/O
  Contract: LayerNorm / RMSNorm forward and backward with fused quantized outputs.

Number formats the pages name but do not define are taken from their public
specifications: OCP 8-bit Floating Point Specification (OFP8) rev. 1.0 for
E4M3, and OCP Microscaling Formats (MX) v1.0 section 6.3 for the E8M0 shared
exponent.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (brute force, closed forms, exhaustive tables, library
routines, invariants). No function is "parity unpinned".
"""

from . import codecs, quant, linear, offsets, grouped, norm  # noqa: F401
