"""CPU oracle of the FLUX-style MMDiT denoising step (test infrastructure).

This package is a plain, slow, readable NumPy statement of what the
denoising step computes: 2x2 latent packing, position ids, 3D RoPE, adaLN
modulated LayerNorm, QK RMSNorm, joint softmax attention, the dual-stream
and single-stream blocks, the conditioning vector, the shifted
flow-matching sigma schedule, the Euler update and the group quantiser.

It is TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it. The product library never
calls it and shares no code with it; the two only receive the same inputs.

Sources (the pages this follows):
  * mflux-rs, "Native Apple Silicon FLUX.1 in Safe Rust": architecture
    cards (Dual-Stream MMDiT, Single-Stream Blocks, 3D RoPE Coordinates,
    Flow-Matching Euler), the RoPE visualiser, the patch packing
    calculator and the accuracy telemetry table.
  * mistral.rs FLUX.1-schnell article, section on FluxStepper and its
    sampling parameters (base/max shift, step counts).
  * stable-diffusion.rs README: quantised weights dequantised inside the
    matmul, 8-bit residual-writing layers with 4-bit elsewhere; the fused
    SDPA / layer_norm / rms_norm kernels it relies on; step caching behind
    a cache threshold (deterministic samplers only).
  * pictor README, numerics section: fp32 accumulation, cosine >= 0.999
    stage gates.

Where the pages leave a formula open, each function states the reading it
takes. Every function is pinned by a CPU test against something other than
itself (closed forms, invariants, brute force, library routines).
"""
from .mmdit import (  # noqa: F401
    pack_latents, unpack_latents, make_ids, rope_frequencies, rope_table,
    apply_rope, layer_norm, modulate, rms_norm, gelu_tanh, silu, linear,
    attention, double_block, single_block, timestep_embedding,
    conditioning_vec, final_layer, step, mu_for_tokens, time_shift,
    schedule, euler_update, quantise, dequantise, pack_int4, unpack_int4,
    bf16_round_up, bf16_rne, quantise_g128, dequantise_g128, pack_g128, unpack_g128,
    rel_l1, cache_decide, new_cache_state, step_cached,
)
