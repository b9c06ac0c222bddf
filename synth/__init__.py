"""Seeded synthetic inputs for the any-precision MoE expert layer.

This package only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no unpacking, no LUT construction, no routing).  Both the
fp64 oracle and the HIP library consume exactly what it produces.

Random stream: every value is a pure function of (seed, tensor id, index)
through the SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), so any single element can be
regenerated without generating the rest.  Normal-like values are Irwin-Hall sums
of twelve 24-bit uniforms, computed exactly, so the host (numpy) and device
(synth_gpu.hip) generators agree bit for bit.

Workloads follow the paper's evaluated MoE shapes (PagedWeight, Section 4,
Table 1: Mixtral-8x7B uses 8 routed experts with top-2 routing) at the sizes
listed in ``CONFIGS``.  Trained weights and datasets are not used: plane words
are uniform random (every parent 8-bit code equally likely), parent LUT rows are
sorted normal(0, 0.02) fp16 values, activations are normal(0, 1) fp16, router
weights normal(0, 0.02) fp16.
"""
from .gen import (  # noqa: F401
    MoEConfig,
    CONFIGS,
    config_by_name,
    u64,
    uniform01,
    normal,
    fp16_normal,
    gen_x,
    gen_router,
    gen_bias,
    gen_planes,
    gen_planes_shape,
    gen_parent_lut_shape,
    gen_aux_fp16,
    gen_aux_u64,
    zipf_ranks,
    gen_parent_lut,
    gen_qmap,
    hot_experts,
    zipf_probs,
    tensor_id,
    TID,
)
