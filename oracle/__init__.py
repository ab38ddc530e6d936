"""CPU oracle of the zero-computation-expert MoE layer.

TEST INFRASTRUCTURE, not part of the product.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import or run
anything in this package.  It shares no code, header, table or helper with the GPU
library in ``mixture_experts_layer_router_amd``; the two meet only through the seeded
inputs of the ``inputs`` package.

Modules:
  moe         vectorised fp64 oracle: router, biased top-K, load, permutation, SwiGLU
              experts, combine (the reference every GPU result is compared against)
  bruteforce  scalar pure-Python formulation for tiny inputs (pins moe)
  dense       dense-masked formulation of the combine (pins moe's permute/combine)
  controller  expert-bias PID controller (one update of the selection bias from loads)
  backward    gradients of the grouped SwiGLU FFN (dx and every expert's dW) for fixed
              picks and gates
  fp8         block-FP8 expert weights: E4M3 encode/decode, power-of-two block scales,
              quantize / dequantize
  tune_routing_inputs
              offline script: tunes the zero-expert bias shift and lists the tokens
              whose selection scores are too close to order reliably; writes
              inputs/routing_tables.json
"""
