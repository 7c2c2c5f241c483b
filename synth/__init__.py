"""Seeded synthetic inputs for the SmolVLA action-expert denoiser.

This package only draws random numbers and lays them out in memory: the
expert's weights (bf16, [out, in] row-major, fixed manifest order), the
per-layer prefix K/V cache (bf16), the prefix language model's weights and
token embeddings (bf16), the prefix pad mask, the Gaussian noise
that starts the flow at t = 1, and the previous-chunk tail used by prefix
overwrite, and the training step's action chunks and flow times.  It holds none of the method's arithmetic and is the only code
that both the CPU oracle and the GPU path consume.
"""
from .gen import (  # noqa: F401
    D_MODEL, N_Q, N_KV, HEAD_DIM, FFN, CHUNK, ACTION_DIM, LM_D_MODEL, LM_FFN,
    WORKLOADS, manifest, weight_count, is_self_layer, lm_manifest, lm_weight_count,
    f32_to_bf16_bits, draw_weights, pack_weights, draw_lm_weights, pack_lm_weights, draw_prefix_embeddings,
    draw_prefix_kv, draw_lengths, make_mask, draw_noise, draw_prev_actions, draw_actions, draw_flow_times,
    make_workload,
)
