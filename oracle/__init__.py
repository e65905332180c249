"""CPU oracle for the block-sparse masked attention forward — TEST INFRASTRUCTURE.

This package is the plain, slow, obviously correct reference that the GPU path
is checked against. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import it. The product path (the C-ABI library and its Python
binding) never imports or calls anything here, and nothing here imports the
product path: the two share no code, headers, tables or constants. The seeded
inputs both sides consume come from the separate `workloads` package.

Everything computes in float64 (numpy), upcasting the exact values the GPU
receives (fp32, or bf16 bit patterns).

Sources (FlexAttention guide = "FlexAttention Guide: Custom Fast Attention in
PyTorch 2.5"; sage2 form = FlashRT-Structures PR #1 "LTX-2.5 attention forms"):
  attention.py  score, score_mod, mask_mod, softmax — guide "The Core Design
                Principles" (score and the two user functions), soft-cap formula
                in "The Problem", ALiBi / window / causal in the "Implementation"
                demo, document and prefix-LM masks in "Production Engineering".
  blockmask.py  tile classification full / empty / partial — guide "Systems
                Mechanics", item 1 (128x128 tile block sparsity).
  quant.py      int8 Q/K and fp8 (OCP E4M3) V quantization — the sage2 form's
                "qk-int8/pv-fp8" description; encodings from the OCP 8-bit
                floating point specification (OFP8, E4M3); the refinements of the
                same PR (finer per-warp Q/K scales, K centering with its delta
                correction).
  brute.py      pure-Python loops on tiny inputs; an independent restatement used
                only to pin attention.py.
  backward.py   dQ, dK, dV and the ALiBi-slope gradient of attention.py's output —
                guide "Systems Mechanics", item 2 (automatic differentiation of the
                score_mod, gradients into learnable slopes); the derivative written
                out by hand. blockmask.transposed_block_mask gives the per-kv-block
                q-block lists a backward walks.

Parity status: every function here is pinned by tests under tests/ marked
"not gpu" (library routines, closed forms, invariants, brute force, values worked
by hand under tests/golden/).
"""
