"""Seeded synthetic inputs for the block-sparse attention forward.

This module draws random numbers and lays out structure (group and document
ids, tensor shapes). It holds none of the attention arithmetic: both the CPU
oracle (through the tests) and the GPU path consume what it returns, so the two
sides always see the same bytes.

Inputs stand in for workloads the pages describe but do not ship:
  * TiRex2 grouped variate attention (TiRex2 PR "perf: expose FlexAttention
    loader override", sections "Context" and "Variate-attention layer"):
    1 target + 16 covariates per group, embedding 512 over 4 heads;
  * document packing with causal masking (FlexAttention guide, "Production
    Engineering", item 1);
  * sliding-window causal GQA with tanh soft-cap (FlexAttention guide,
    "Implementation" demo and "The Problem" soft-cap formula);
  * long dense self-attention at S=24576 over 32 heads, run in bf16 and in the
    int8-QK / fp8-PV form (FlashRT-Structures PR #1, the sage2 attention form).

Random draws use numpy's PCG64 (`numpy.random.default_rng(seed)`) in a fixed
order: structure, Q, K, V, then the V channel scales.
"""
from .synth import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    decode_workload,
    f32_to_bf16_bits,
    grad_output,
    grouped_sweep,
    make_workload,
    random_case,
    SWEEP_GROUPS,
    WORKLOADS,
)
