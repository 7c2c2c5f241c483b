/*
 * smolexp — the SmolVLA action-expert denoising loop on AMD Instinct MI355X (gfx950).
 *
 * Given the VLM's per-layer prefix K/V cache and its pad mask, the library runs
 * the flow-matching action head: starting from Gaussian noise at t = 1 it takes
 * n_steps explicit Euler steps x <- x + dt * v(x, t) toward t = 0, where the
 * velocity v comes from a stack of width-720 transformer layers over the
 * 50 x 32 action chunk; even layers self-attend over [valid prefix ; causal
 * chunk], odd layers cross-attend to the valid prefix (noeira docs "SmolVLA",
 * Architecture: table rows "Action expert" and "Action head", the paragraph on
 * the query (prefix once, expert ten times), the flow-matching objective and
 * the block attention mask).
 *
 * Conventions for every entry point:
 *  - Return 0 on success or a negative SMOLEXP_E_* code.  All argument checks
 *    run on the host before anything is enqueued; a failed check enqueues
 *    nothing.  smolexp_strerror() names a code, smolexp_last_error() gives
 *    the handle's last detailed message.
 *  - "device" pointers are HIP device memory on the handle's device; "host"
 *    pointers are ordinary host memory.  The library never frees or keeps a
 *    caller pointer beyond the work it enqueues.
 *  - Device contents are not checked: NaN in gives NaN out.
 *  - A handle is not re-entrant: use one handle per concurrent stream.
 *  - No environment variable changes the library's behaviour.
 */
#ifndef SMOLEXP_H
#define SMOLEXP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct smolexp_handle* smolexp_t;

enum {
  SMOLEXP_OK = 0,
  SMOLEXP_E_INVAL = -1,  /* null pointer, size out of range, unsupported config */
  SMOLEXP_E_STATE = -2,  /* call out of order (e.g. denoise before load_weights) */
  SMOLEXP_E_SIZE = -3,   /* weight buffer length != smolexp_weight_count(cfg) */
  SMOLEXP_E_NOMEM = -4,  /* device or host allocation failed */
  SMOLEXP_E_HIP = -5     /* HIP runtime or launch error; see smolexp_last_error */
};

/*
 * Configuration, fixed at create.  The architecture fields must equal the
 * SmolVLA expert's (d_model 720, 15 query heads over 5 KV heads of dim 64,
 * SwiGLU width 2048, chunk 50, action width 32); other values return
 * SMOLEXP_E_INVAL.  n_layers may be 1..64 (16 in SmolVLA; layer l self-attends
 * when l is even).  n_steps is 1..64 (10 in SmolVLA).  rope_theta, rms_eps and
 * the time-embedding periods are readings the pages leave open; defaults are
 * 10000, 1e-6, 4e-3 and 4.0.
 */
typedef struct smolexp_config {
  int n_layers;
  int d_model;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  int ffn;
  int chunk;
  int action_dim;
  int n_steps;
  int max_batch;     /* 1..1024: largest batch a call may pass */
  int max_prefix;    /* 1..4096: largest padded prefix length P a call may pass */
  float rope_theta;
  float rms_eps;
  float t_min_period;
  float t_max_period;
  int use_graphs;    /* 1: capture each call's launch sequence once and replay it as a HIP graph */
  int batch_groups;  /* 0..8: a call's queries run as this many groups whose loops proceed
                        concurrently (on side streams of default priority, or as parallel
                        branches of the graph); 0 = automatic (two groups from 64
                        queries on, one per 64 queries from 192 on).
                        Every group but the last holds a multiple of 8 queries.  The results
                        of a query depend on the size of its group only within the tolerances,
                        as for any change of batch composition. */
  int weight_format; /* SMOLEXP_WEIGHTS_FP16 (0, the default) or SMOLEXP_WEIGHTS_E4M3 (an explicit
                        opt-in, batches of at most 8 queries: max_batch 1..8).  See
                        smolexp_load_weights. */
} smolexp_config;

/* Storage of the streamed weight matrices.  PyPI "mlx-smolvla", Run a checkpoint: 8-bit and
 * 4-bit weight presets exist only as explicit opt-ins; dense weights stay the default. */
enum {
  SMOLEXP_WEIGHTS_FP16 = 0, /* every bf16 value re-encoded exactly (fp16, a power-of-two scale per matrix) */
  SMOLEXP_WEIGHTS_E4M3 = 1  /* OCP FP8 E4M3 codes, one power-of-two scale per output row
                               (smolexp_quantize_e4m3_rows): half the bytes, rounded weights */
};

/* Fill *cfg with the SmolVLA expert (16 layers, 10 steps, max_batch 128, max_prefix 512). Host only. */
void smolexp_default_config(smolexp_config* cfg);

/*
 * Number of bf16 weight elements smolexp_load_weights expects for cfg
 * (98,210,912 for 16 layers; 25,755,872 for 4), or 0 if cfg is invalid.
 * Host only; needs no GPU.
 */
size_t smolexp_weight_count(const smolexp_config* cfg);

/*
 * The flow times the loop uses, host only: dt = fl32(-1/n_steps),
 * t_0 = 1, t_{k+1} = fl32(t_k + dt), exactly n_steps values (noeira docs
 * "SmolVLA", Architecture: from t = 1 toward t = 0).  t_out has room for
 * cfg->n_steps floats; dt_out may be NULL.
 */
int smolexp_schedule(const smolexp_config* cfg, float* t_out, float* dt_out);

/*
 * How a call of `batch` queries is split into concurrent groups (cfg->batch_groups):
 * returns the number of groups (1..8) and, when sizes is not NULL, writes the queries of
 * each group in call order (sizes has room for 8).  SMOLEXP_E_INVAL for an invalid cfg or
 * batch outside 1..max_batch.  Host only; needs no GPU.
 */
int smolexp_batch_groups(const smolexp_config* cfg, int batch, int* sizes);

/*
 * Quantize a row-major [rows][cols] float64 matrix to OCP 8-bit floating point E4M3 (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite value 448, no
 * infinities) with one scale per row, as smolexp_load_weights does for
 * SMOLEXP_WEIGHTS_E4M3 (the pages name 8-bit presets, PyPI "mlx-smolvla", Run a checkpoint,
 * but no format; this is the reading taken).  Row r's scale is the power of two
 * 2^e, e the smallest integer with max_k |w[r][k]| / 2^e <= 448 (1 for an all-zero row), and
 * codes[r][k] is the E4M3 code nearest to w[r][k] / 2^e, ties to even; the code value times
 * scales[r] is the weight's 8-bit value.  codes: rows x cols bytes (caller-owned),
 * scales: rows floats.  SMOLEXP_E_INVAL for NULL buffers, negative sizes, a value that is
 * not finite, or a row whose scale would fall outside float's normal range (2^-126 .. 2^127);
 * the outputs are then unspecified.  Host only; needs no GPU.
 */
int smolexp_quantize_e4m3_rows(const double* w, int rows, int cols, uint8_t* codes, float* scales);

/*
 * Create a handle on HIP device hip_device: validates cfg, allocates the
 * workspace for max_batch x max_prefix and the weight store, and builds the
 * RoPE table.  *out is set only on success.  Release with smolexp_destroy.
 */
int smolexp_create(const smolexp_config* cfg, int hip_device, smolexp_t* out);

/*
 * Load the expert's weights from one flat host buffer of bf16 bit patterns in
 * manifest order, every matrix row-major [out, in] (the nn.Linear layout,
 * noeira docs "SmolVLA", Weights):
 *   action_in.w [720,32], action_in.b [720], time_in.w [720,1440],
 *   time_in.b [720], time_out.w [720,720], time_out.b [720];
 *   per layer l: norm1.g [720], q.w [960,720], (l even only: k.w [320,720],
 *   v.w [320,720]), o.w [720,960], norm2.g [720], gate.w [2048,720],
 *   up.w [2048,720], down.w [720,2048];
 *   final_norm.g [720], action_out.w [32,720], action_out.b [32].
 * n_elems must equal smolexp_weight_count (else SMOLEXP_E_SIZE).  The data is
 * copied (matrices re-encoded exactly as fp16 with a power-of-two scale per
 * matrix; RMSNorm gains folded into the matrix that follows; action_in folded
 * into the action half of time_in, whose product with it is a weight-only
 * [720,32] matrix, rounded once to fp16, plus a bias term), and the time
 * vectors of the configured schedule are computed; the caller may free
 * bf16_host on return.  Synchronous.
 * With weight_format SMOLEXP_WEIGHTS_E4M3 every matrix the loop streams is stored as the
 * loop applies it (gains folded; the [720,32] product formed in float64) and quantized by
 * rows (smolexp_quantize_e4m3_rows); the time-embedding half of time_in, which meets only
 * the fixed flow times, and the biases stay exact.  SMOLEXP_E_INVAL if a row cannot be
 * quantized.  The prefill and the training step do not read these matrices.
 */
int smolexp_load_weights(smolexp_t h, const uint16_t* bf16_host, size_t n_elems);

/*
 * Denoise a batch of action chunks (the whole loop, asynchronous on hip_stream;
 * NULL = the null stream).  noeira docs "SmolVLA", Architecture: a query's
 * prefix is run once and its per-layer keys/values cached, then the expert is
 * evaluated once per Euler step (ten times) on the chunk, from noise at t = 1
 * toward t = 0; the block attention mask keeps the prefix blind to the actions,
 * which is why the cached prefix suffices.
 *   prefix_kv    device bf16, [n_layers][2 (K, V)][batch][5][prefix_len][64]:
 *                each layer's cached prefix keys (already rotated at their
 *                prefix positions) and values.  Read only.
 *   prefix_mask  device uint8 [batch][prefix_len], nonzero = valid token; any
 *                pattern.  Chunk row i of query b sits at RoPE position
 *                (number of valid tokens of b) + i.  Masked tokens are left out
 *                of every softmax (their K/V may hold anything, NaN included).
 *                A query with no valid token gets zero cross-attention output.
 *   prefix_len   P, 1..max_prefix.
 *   noise        device fp32 [batch][50][32]: x at t = 1.  Read only.
 *   out_actions  device fp32 [batch][50][32]: x after the last step.
 *   batch        1..max_batch.
 * The library's workspace is in use until the stream work completes.
 */
int smolexp_denoise(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask,
                    int prefix_len, const float* noise, float* out_actions, int batch,
                    void* hip_stream);

/*
 * smolexp_denoise for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * kernels and launches as smolexp_denoise (launched directly, never through a
 * cached graph), but the per-call activations live in a fixed array of device
 * memory inside the library (one copy per GPU, about 12.5 MB, held until the
 * process ends) instead of the handle's workspace; the handle's weights and
 * tables are only read.  The call allocates nothing: no hipMalloc, no graph.
 *   batch  1..16 (and <= the handle's max_batch); larger batches return
 *          SMOLEXP_E_INVAL ("batch above the no-alloc workspace's maximum").
 * Other arguments and errors as for smolexp_denoise.  Every call on one GPU
 * shares that GPU's array, from any handle: calls that overlap on one GPU (on
 * two streams, or from two threads) race and give undefined results; calls
 * ordered on one stream are safe.  The array keeps the last call's contents
 * (what must start at zero is cleared by each call).
 */
int smolexp_denoise_noalloc(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask,
                            int prefix_len, const float* noise, float* out_actions, int batch,
                            void* hip_stream);

/*
 * Options for smolexp_denoise_ex.  Every field may be zero/NULL.
 *   prev_actions    device fp32 [batch][overwrite_rows][32]: tail of the
 *                   previous chunk for prefix overwrite ("Paper vs hardware 11:
 *                   SmolVLA", What I ran).  Before every step k, chunk rows
 *                   i < overwrite_rows are set to t_k*noise_i + (1-t_k)*prev_i,
 *                   the flow-matching path point at t_k (noeira docs "SmolVLA",
 *                   flow-matching objective).  Required when overwrite_rows > 0.
 *   overwrite_rows  d, 0..50.
 *   out_velocities  device fp32 [n_steps][batch][50][32] or NULL: v at each step.
 *   out_states      device fp32 [n_steps][batch][50][32] or NULL: x after each step.
 *   out_status      device int [1] or NULL: the call's status word, 0 when every
 *                   activation rounded to fp16 for the matrix cores stayed inside
 *                   fp16's range; otherwise SMOLEXP_RANGE_* bits name what left it
 *                   (it became infinite, and the call's results are not valid).
 *                   Written by the call's kernels (cleared by its first one); read
 *                   it after the stream work completes.
 */
typedef struct smolexp_denoise_opts {
  const float* prev_actions;
  int overwrite_rows;
  float* out_velocities;
  float* out_states;
  int* out_status;
} smolexp_denoise_opts;

/*
 * Bits of a call's status word (smolexp_denoise_opts.out_status).  The GEMM operands are
 * fp16 (largest finite value 65504); an activation of larger magnitude cannot be
 * represented there.  The library detects this instead of scaling: values that large do
 * not occur with SmolVLA-scale weights (the residual stream stays orders of magnitude
 * below), and a checkpoint that produced them would need its own scaling.
 */
enum {
  SMOLEXP_RANGE_RESIDUAL = 1,   /* the fp16 copy of the residual stream (also a prefill's embeddings) */
  SMOLEXP_RANGE_FFN = 2,        /* the SwiGLU output */
  SMOLEXP_RANGE_ATTENTION = 4,  /* an attention output */
  SMOLEXP_RANGE_TIME = 8        /* the time MLP's hidden layer, or the Euler state */
};

/* smolexp_denoise with options (opts may be NULL = none). */
int smolexp_denoise_ex(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask,
                       int prefix_len, const float* noise, float* out_actions, int batch,
                       void* hip_stream, const smolexp_denoise_opts* opts);

/*
 * One evaluation of the velocity field v(x, t | prefix) (the expert's forward
 * pass, no Euler update; noeira docs "SmolVLA", Architecture: the expert maps
 * the noisy chunk at flow time t, the time embedding and the cached prefix to a
 * velocity, whose training target is eps - a).  x and out_v are device fp32 [batch][50][32]; the other
 * arguments are as for smolexp_denoise.  Used to check a single step against
 * an oracle on the oracle's own x.  Asynchronous on hip_stream.
 */
int smolexp_velocity(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask,
                     int prefix_len, const float* x, float t, float* out_v, int batch,
                     void* hip_stream);

/*
 * Prefix prefill: the step before the denoising loop, which fills the per-layer
 * K/V cache that smolexp_denoise reads (noeira docs "SmolVLA", Architecture: the
 * language model, SmolLM2, 16 layers of width 960 with grouped-query attention of
 * 15 query heads over 5 KV heads of dim 64, RoPE, SwiGLU and RMSNorm, run once
 * over the prefix; the block attention mask keeps the prefix from seeing the
 * actions).  The handle's n_layers language-model layers fill n_layers cache
 * layers.  Readings where the pages are silent: the prefix attends to itself in
 * both directions (one block of the mask), pads are not keys; a token's RoPE
 * position is the number of valid tokens before it (the chunk continues at
 * n_valid + i), with the handle's rope_theta and rms_eps; SwiGLU width 2560; no
 * biases.
 *
 * smolexp_lm_weight_count: elements of the language model's flat bf16 buffer,
 * 9,832,320 per layer (0 for an invalid config).
 *
 * smolexp_load_lm_weights: bf16 bit patterns in manifest order, every matrix
 * row-major [out, in]; per layer l: norm1.g [960], q.w [960,960],
 * k.w [320,960], v.w [320,960], o.w [960,960], norm2.g [960],
 * gate.w [2560,960], up.w [2560,960], down.w [960,2560].  Copied and re-encoded
 * as for smolexp_load_weights; n_elems must equal smolexp_lm_weight_count (else
 * SMOLEXP_E_SIZE).  Synchronous.
 *
 * smolexp_prefill (asynchronous on hip_stream; NULL = the null stream):
 *   prefix_emb   device bf16 [batch][prefix_len][960]: the prefix token
 *                embeddings (vision connector output, text embeddings, the
 *                state token).  Read only.  Masked rows may hold anything.
 *   prefix_mask  device uint8 [batch][prefix_len], nonzero = valid token.
 *   out_kv       device bf16 [n_layers][2 (K, V)][batch][5][prefix_len][64]:
 *                written; K after the rotation at each token's position.  This
 *                is smolexp_denoise's prefix_kv.  Rows of masked tokens are
 *                written but unspecified (they are never attended).
 * The library keeps a workspace for batch x prefix_len rows; a call with more
 * rows than any before it grows that workspace first, which synchronizes the
 * device.  SMOLEXP_E_STATE before smolexp_load_lm_weights; SMOLEXP_E_INVAL for
 * NULL pointers or batch / prefix_len outside 1..max_batch / 1..max_prefix.
 */
size_t smolexp_lm_weight_count(const smolexp_config* cfg);
int smolexp_load_lm_weights(smolexp_t h, const uint16_t* bf16_host, size_t n_elems);
int smolexp_prefill(smolexp_t h, const void* prefix_emb, const uint8_t* prefix_mask, int prefix_len,
                    void* out_kv, int batch, void* hip_stream);

/*
 * Flow-matching training step of the expert: the loss of one batch and the
 * gradient of every expert tensor (noeira docs "SmolVLA", Architecture: the
 * fine-tuning objective, x_t = t eps + (1 - t) a and the squared error of
 * v_theta(x_t, t | prefix) against eps - a; Fine-tuning: only the expert trains,
 * so the prefix K/V is a frozen input).  Readings where the pages are silent:
 * the loss is the mean over the batch's B x 50 x 32 elements; t and eps are
 * drawn by the caller; no optimizer update is applied.  The weights are those of
 * the last smolexp_load_weights (the library keeps them as given, bf16).
 *   prefix_kv, prefix_mask, prefix_len  as for smolexp_denoise (read only).
 *   actions    device fp32 [batch][50][32]: the target chunks a.  Read only.
 *   noise      device fp32 [batch][50][32]: eps.  Read only.
 *   t          device fp32 [batch]: each query's flow time.  Read only.
 *   out_grads  device fp32 [smolexp_weight_count]: written (not accumulated),
 *              d loss / d weight in manifest order, one value per weight.
 *   out_loss   device fp32 [1]: written.
 * Precision: matrix products take bf16 operands with fp32 accumulation; norms,
 * softmax, the loss and the residual stream are fp32; activations that only
 * feed products are kept in bf16, as the products read them.
 * Deterministic (no atomics).  The library keeps a workspace of about 41 KB per
 * chunk row per layer (the activations) for the largest batch x prefix_len
 * seen; a call that needs more grows it first, which synchronizes the device
 * and drops the handle's cached graphs.  With use_graphs the launch sequence is
 * captured once per call signature (pointers, batch, prefix_len) and replayed,
 * as for smolexp_denoise.  Asynchronous on hip_stream otherwise.  SMOLEXP_E_STATE before
 * smolexp_load_weights; SMOLEXP_E_INVAL for NULL pointers or batch /
 * prefix_len out of range.
 */
int smolexp_train_step(smolexp_t h, const void* prefix_kv, const uint8_t* prefix_mask, int prefix_len,
                       const float* actions, const float* noise, const float* t, float* out_grads,
                       float* out_loss, int batch, void* hip_stream);

/*
 * Measurement hook: average duration in microseconds of one launch of one
 * kernel of the loop, timed with HIP events on hip_stream (synchronous) around
 * `reps` (1..100000) back-to-back launches.  Launch i repeats the (i mod n)-th
 * launch of that kernel in the first step of the last call (n = one per layer
 * that uses it), so the weights change from launch to launch as in the loop.
 * With graphs enabled the launches are captured as one HIP graph, replayed once
 * untimed and once timed.  It reuses the workspace contents of the last
 * smolexp_denoise/_ex call, which must have used the same batch and
 * prefix_len, and leaves that workspace's numbers unspecified.
 *   kernel: 0 = self-attention layer QKV projection, 1 = self attention,
 *           2 = cross attention (with the layer's Q projection at batch <= 8),
 *           3 = o projection, 4 = gate/up projection, 5 = down projection,
 *           6 = action_out + Euler update, 7 = the whole loop (one
 *           smolexp_denoise call), 8 = cross-attention layer Q projection
 *           (its own launch above batch 8; at batch <= 8 it is part of
 *           kernel 2 and this id returns SMOLEXP_E_STATE), 9 = the time MLP's
 *           first layer (action_in folded in) + SiLU, 10 = the time MLP's
 *           second layer into the residual stream.
 * SMOLEXP_E_INVAL for other ids, SMOLEXP_E_STATE without a previous call or
 * for a kernel that call did not launch.
 */
int smolexp_time_kernel(smolexp_t h, int kernel, int reps, void* hip_stream, float* avg_us);

/* Static name of an error code. */
const char* smolexp_strerror(int code);

/* Last error message recorded on h ("" if none); valid until the next call on h. */
const char* smolexp_last_error(smolexp_t h);

/* Free everything h owns (waits for its device work first).  NULL is ignored. */
void smolexp_destroy(smolexp_t h);

#ifdef __cplusplus
}
#endif

#endif /* SMOLEXP_H */
