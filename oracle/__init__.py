"""CPU oracle for one GPU's share of an expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls, links or executes anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.  It
shares no code with the HIP path: no kernels, no headers, no helpers, no tables.

The oracle is plain and slow on purpose.  Floating point work is done in fp64,
except where a step makes a decision that the method fixes in a narrower type
(the FP8 requantisation of the SwiGLU output, which is decided in fp32 on both
sides).  Each function cites the passage it follows:

  [NVLinkOneSided, Abstract]  "One-Sided Expert-Parallel All-to-All for
      Mixture-of-Experts Inference over NVLink" (wpnews.pro summary of
      arXiv 2611.13188v1), abstract paragraph.
  [Relay-free Ascend, Abstract]  "Relay Buffer Independent Communication over
      Pooled HBM for Efficient MoE Inference on Ascend" (mlsanity.com entry for
      arXiv 2605.06055), section "Abstract (arXiv)".
  [GC-MoE feed, Full text]  "GC-MoE: Overlapping Expert-Parallel Token Dispatch
      with FP8/FP4 Grouped GEMM via CUDA Green Contexts" (Astral Feed entry for
      arXiv 2611.04222v1), section "Full text".
  [GC-MoE explainer, <section>]  "GC-MoE: Decoupling MoE Communication and
      Computation with CUDA Green Contexts" (kongchang.com), by section title.

Modules:
  codecs  -- FP8 e4m3 (OCP), FP4 e2m1, e8m0, bf16 encode/decode from the format
             definitions.
  gating  -- softmax over the top-k logits.
  layer   -- rank-major dispatch, block-scale dequantisation, expert SwiGLU FFN,
             1x128 FP8 requantisation, weighted combine, and the whole layer.
"""
