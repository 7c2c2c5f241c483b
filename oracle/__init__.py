"""CPU oracle for the SmolVLA action-expert denoising loop.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code that states what
the denoiser computes, one query at a time, in the order the method does it.
Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import it.  The GPU library never calls it and shares no code with it; the
two meet only through the seeded inputs of the ``synth`` package.

Sources (page title, then section):
  * noeira docs "SmolVLA", Architecture: the expert has 16 layers of width
    720, even layers self-attend and odd layers cross-attend to the VLM's
    cached keys/values; 10 Euler steps from Gaussian noise at t = 1 toward
    t = 0; chunk of 50; the prefix is computed once, the expert ten times;
    the flow-matching path x_t = t*eps + (1 - t)*a with target eps - a; the
    block attention mask (the prefix never sees the actions); 32-wide
    padded action vectors.
  * "Paper vs hardware 11: SmolVLA", What the paper claims: causal
    self-attention over the chunk, cross-attention to the VLM keys/values,
    conditional flow matching, chunk 50; What I ran: prefix overwrite of the
    first d ~ 7 chunk rows at chunk boundaries.
  * noeira docs "SmolVLA", Architecture table, language-model row:
    grouped-query attention 15/5 heads of dim 64, RoPE, SwiGLU, RMSNorm
    (the expert uses the same block family at width 720).
  * CSDN "SmolVLA PyTorch official-like 精度排查过程与结论", sections 8 and 12:
    K/V cache in bf16, Euler update and output in fp32, bf16 values used with
    fp32 storage ("fake bf16").  The oracle decodes every bf16 input exactly
    and computes in float64.

Where the pages leave a step open, the reading taken (layer parity, RoPE
pairing and theta, RMSNorm epsilon, time-embedding form, concat order, biases,
mask semantics, schedule rounding, overwrite timing) is stated at the
function that implements it.

Pins (what fixes each function other than itself; all in tests/):
  rms_norm ........ closed form on constant rows; torch.nn.functional.rms_norm
  silu ............ closed values; torch.nn.functional.silu
  rope ............ identity at position 0; unit-vector rotation closed form;
                    norm preservation; scores depend only on position offset
  time_embedding .. e(0) = [0..0, 1..1]; sin^2 + cos^2 = 1; quarter-period
                    closed values
  attention ....... float64 triple-loop brute force on tiny shapes; one valid
                    key returns that V row; equal keys give the mean of V;
                    torch scaled_dot_product_attention with GQA and a mask
  embed ........... closed forms with degenerate weights: the time path alone
                    (time_in = [0 | I]) and the action path alone (time_in =
                    [I | 0], a selector action_in), and the action path pushed
                    through identity layers and the head; copies of embed with
                    a planted mistake (swapped concatenation, SiLU after
                    time_out, a dropped b_in or b_t1) fail them
  expert layer .... composition of torch library routines (rms_norm, linear,
                    scaled_dot_product_attention(enable_gqa), silu) with a
                    complex-number rotary embedding
  expert (whole) .. chunk causality, pad invariance (NaN pads), batch
                    invariance, block-mask joint-pass equivalence, and
                    degenerate-weight closed forms of the whole loop; its own
                    rounding (activations held in float32 move the velocity
                    by < 1e-5 relative, far below the 1e-2 tolerance)
  schedule/Euler .. closed-form trajectories under stub velocity fields
                    (constant, linear, straight flow-matching path)
  overwrite ....... closed form under v = 0; fixed point on the straight path
  prefill (prefill.py: the prefix language model's per-layer keys/values)
    layer ......... composition of torch library routines (rms_norm, linear,
                    scaled_dot_product_attention(enable_gqa) with the key
                    mask, silu), complex-number rotary embedding, positions
                    from torch's cumulative sum
    positions ..... closed values
    whole prefill . NaN-pad invariance; removing the pads leaves the valid
                    tokens' keys/values unchanged; bidirectional within the
                    prefix (layer-1 keys of token 0 depend on the last token,
                    layer-0 keys do not); one-token closed form; batch layout
    bf16 rounding . closed values (ties to even, subnormals)
  training step (train.py: the flow-matching loss and the expert's weight gradients)
    per-op derivatives  central finite differences (SiLU, RMSNorm, masked
                    attention with empty and single-key rows); the rotary
                    backward is the transpose (adjoint identity)
    whole step .... central finite differences of the float64 batch loss along
                    a random direction in every manifest tensor; torch autograd
                    through a composition of torch library routines; closed
                    form with a zero action_out matrix; the forward's velocity
                    is expert.velocity's; query shares add up to the batch
  8-bit weights (quant.py: E4M3 codes with per-row power-of-two scales, and the expert
  with its streamed matrices quantized)
    e4m3 .......... the format's code points (largest finite, smallest normal and
                    subnormal, NaN); every code round-trips; exhaustive nearest-value
                    search with ties to even; torch's float8_e4m3fn cast; the rounding
                    error bound
    row scales .... powers of two putting each row's max in (224, 448]
    streamed model  without rounding it is the float64 expert (to float64 rounding);
                    copies with a planted mistake (a gain not folded, the time half
                    dropped) fail that; quantized matrices sit on their rows' grid
No function is left parity unpinned.
"""
from .expert import (  # noqa: F401
    bf16_bits_to_float, decode_weights, rms_norm, silu, rope, time_embedding,
    attention, embed, expert_layer, head, velocity, ExpertConfig,
)
from .flow import schedule, overwrite_rows, euler_denoise, denoise_query, denoise_batch  # noqa: F401
from . import quant  # noqa: F401
from .prefill import (  # noqa: F401
    PrefillConfig, prefix_positions, prefill_layer, prefill, prefill_batch, round_to_bf16_bits,
)
from .train import (  # noqa: F401
    silu_grad, linear_bwd, rms_norm_bwd, rope_bwd, attention_bwd, query_loss_and_grads, train_batch,
)
