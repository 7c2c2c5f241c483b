// Internal declarations shared by the host API (smolexp_api.cpp) and the HIP
// kernels (kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smolexp {

// SmolVLA action-expert shapes (noeira docs "SmolVLA", Architecture table).
constexpr int kD = 720;        // model width
constexpr int kHQ = 15;        // query heads
constexpr int kHKV = 5;        // key/value heads
constexpr int kHD = 64;        // head dim
constexpr int kFFN = 2048;     // SwiGLU width
constexpr int kChunk = 50;     // actions per chunk
constexpr int kAD = 32;        // padded action width
constexpr int kNQ = kHQ * kHD;         // 960
constexpr int kNKV = kHKV * kHD;       // 320
constexpr int kNQKV = kNQ + 2 * kNKV;  // 1600
constexpr int kGU = 2 * kFFN;          // 4096 (gate and up, interleaved in 16-row blocks)
constexpr int kMaxSteps = 64;
constexpr int kMaxLayers = 64;
// The prefix language model that fills the per-layer K/V cache (SmolLM2 layers: width 960,
// the same 15 / 5 heads of dim 64; the SwiGLU width is not on the pages, 2560 is SmolLM2-360M's).
constexpr int kLmD = 960;
constexpr int kLmFFN = 2560;
constexpr int kLmGU = 2 * kLmFFN;      // 5120 (gate and up, interleaved in 16-row blocks)

typedef _Float16 half_t;
typedef uint16_t bf16_t;       // bf16 bit pattern

// Blocked layout of every GEMM operand (weights [N][K] and the fp16
// activations [M][K]): 16-row x 8-column micro-tiles of 256 bytes, row block
// major, so element (r, k) of a matrix stored with KC = K / 8 column chunks
// sits at ((r / 16) * KC + k / 8) * 128 + (r % 16) * 8 + k % 8.  The 16 rows
// of one chunk are contiguous, which is exactly what one MFMA fragment load
// (lane l: row l % 16, chunk l / 16) reads: four 256-byte runs, 1 KB in a row.
// Row counts are padded to a multiple of 16.
__host__ __device__ inline size_t t16_off(int r, int k, int kc) {
  return ((size_t)(r >> 4) * kc + (k >> 3)) * 128 + (r & 15) * 8 + (k & 7);
}
// The fp32 residual stream uses the same idea with 16-row x 4-column tiles:
// element (r, k) with K4 = K / 4 column chunks at ((r / 16) * K4 + k / 4) * 64 + (r % 16) * 4 + k % 4.
__host__ __device__ inline size_t t32_off(int r, int k, int k4) {
  return ((size_t)(r >> 4) * k4 + (k >> 2)) * 64 + (r & 15) * 4 + (k & 3);
}

// A-operand sources of the GEMM.
enum AMode : int {
  A_F16 = 0,    // fp16, blocked (t16_off), lda = stored K (multiple of 8)
  A_NORM = 1,   // fp16(h), blocked, lda = 768: RMSNorm'd with the gain folded into W and the row
                // scale 1/rms applied to the sums; each kernel sums the squares of the rows it
                // streams (fp16 values)
  A_X = 2,      // fp32 Euler state, row-major [M][32]; prefix overwrite applied on load
};

// GEMM epilogues.
enum EMode : int {
  E_TIMEIN = 1,    // out16 = SiLU(acc + cvec)                (action_in + time MLP, first layer)
  E_H_BIAS = 2,    // h = acc + bias; h16 = fp16(h)           (time MLP, second layer)
  E_H_RESID = 3,   // h += acc; h16 = fp16(h)                 (o and down projections)
  E_QKV = 4,       // RoPE on Q and K, scatter to Q/Kc/Vc bf16 (attention input)
  E_SWIGLU = 5,    // out16 = SiLU(gate) * up                 (FFN)
  E_ACTOUT = 6,    // v = acc + bias; x += dt * v             (action_out + Euler)
  E_PF_QKV = 7,    // as E_QKV with `seq` rows per query: Q, and K/V into the cache (prefill)
  E_PF_RESID = 8,  // as E_H_RESID at the prefix model's width (960 stored columns)
};

// Bits of a call's status word: an activation that is rounded to fp16 for the matrix cores
// (largest finite value 65504) was beyond that range, so it became infinite and the results are
// not valid.  Set by the kernel that rounds it (atomicOr), cleared by the call's first kernel.
constexpr int kRangeResidual = 1;   // the fp16 copy of the residual stream (RMSNorm'd products)
constexpr int kRangeFfn = 2;        // the SwiGLU output
constexpr int kRangeAttention = 4;  // the attention output
constexpr int kRangeTime = 8;       // the time MLP's hidden layer, or the Euler state as its operand

struct GemmArgs {
  int M, N, K;
  int* status;          // the call's status word (kRange* bits), or nullptr
  const void* A;
  int lda;
  // A_NORM
  float inv_k;
  float eps;
  // A_X
  float* x;
  const float* noise;
  const float* prev;
  int ow_rows;
  float t;
  // weights: fp16 [N][K] blocked (t16_off) with ldw = stored K, values scaled by 1 / w_scale;
  // or, when wrs is not nullptr, OCP E4M3 codes (one byte per element, the same element
  // offsets) with real value = code value * wrs[n] (one power of two per stored row)
  const half_t* W;
  int ldw;
  float w_scale;
  const float* wrs;
  // epilogue
  const float* bias;   // bias, or the per-step time vector for E_TIMEIN
  half_t* out16;       // fp16 activations, blocked (t16_off), ldo = stored K
  int ldo;
  float* h;            // fp32 residual stream, blocked (t32_off), K = 720
  half_t* h16;         // its fp16 copy, blocked (t16_off), 768 stored columns (720.. stay zero)
  bf16_t* q;            // [B][15][seq][64]
  bf16_t* kc;           // [B][5][seq][64]: the chunk's K (E_QKV), a cache layer's K (E_PF_QKV)
  bf16_t* vc;
  int seq;              // rows per query (E_PF_QKV; E_QKV: the chunk, 50)
  const float2* ropeq;  // [row][32] (cos, sin) of each row's position
  float dt;
  float* vel_out;
  float* st_out;
  float* final_out;
};

struct AttnArgs {
  int* status;           // the call's status word (kRangeAttention), or nullptr
  const bf16_t* q;       // [B][15][seq][64]
  const bf16_t* kc;      // [B][5][50][64] (self only)
  const bf16_t* vc;
  const bf16_t* pk;      // this layer's prefix K: [B][5][P][64]
  const bf16_t* pv;      // this layer's prefix V
  const uint8_t* mask;   // [B][P]
  half_t* out;           // [B*seq][960] fp16, blocked (t16_off)
  int B, P;
  int seq;               // query rows per query head: the chunk (50), or the prefix (P) in a prefill
  // cross layers of a small batch (use_cross_q): the query projection runs in the
  // attention launch.  wq = the layer's Q weight ([960][768] blocked, RMSNorm gain
  // folded, values scaled by 1 / w_scale); h16 = fp16 residual [B*50][768] blocked.
  // wq == nullptr: Q comes from q.
  const half_t* wq;
  int ldw;
  float w_scale;
  const float* wrs;      // not nullptr: wq holds E4M3 codes with these row scales (as GemmArgs)
  const half_t* h16;
  float inv_k, eps;
  const float2* ropeq;
};
constexpr int kCrossQMaxBatch = 8;
bool use_cross_q(int B);  // the cross layers of this batch size fold the Q projection into attention

struct PrologueArgs {
  int* status;             // cleared to 0 (when not nullptr)
  int B;                   // queries (0: time vectors only)
  int n_t;                 // number of flow times whose time vectors are computed (0: none)
  float t[kMaxSteps];
  const uint8_t* mask;     // [B][P]
  int P;
  const float2* rope;      // [pos][32] (cos, sin) by position
  float2* ropeq;           // out [B*50][32]: the rows of rope at positions n_valid(b) + i
  const float* x_in;       // [B][50][32]
  float* x;                // out: Euler state
  const half_t* w_t1e;     // time_in weight, its time-embedding half [720][720] row-major (fp16, scaled)
  float s_t1;
  const float* b_t1;
  float* cvec;             // out [n_t][720] = W_t1[:, 720:] e(t) + b_t1
  const double* inv_period;  // [360] 1 / p_i of the time embedding
};

// Per-call activations of the denoising loop (device memory): the Euler state x, the fp32
// residual h and its fp16 copy h16 (768 stored columns, 720.. zero), the time MLP's hidden
// layer s16, the attention output o16, the SwiGLU output u16, the chunk's Q / K / V, the
// RoPE rows of each chunk row, and a second Euler-state buffer x2 (the step-boundary launch
// reads step k's state from one of x, x2 and writes step k + 1's to the other: several of its
// workgroups read each state row).  Blocked operands hold whole 16-row blocks.
struct CallWs {
  float* x;
  float* h;
  half_t *s16, *o16, *u16, *h16;
  bf16_t *q, *kc, *vc;
  float2* ropeq;
  float* x2;
};
constexpr size_t ws_align256(size_t n) { return (n + 255) & ~(size_t)255; }
// Sizes of the CallWs buffers, in the order they are carved, for max_batch queries.
constexpr int kCallWsParts = 11;
constexpr size_t call_ws_part(int max_batch, int i) {
  const size_t M = (size_t)max_batch * kChunk, Mp = (M + 15) & ~(size_t)15;
  const size_t sz[kCallWsParts] = {M * kAD * 4,  Mp * kD * 4,    Mp * kD * 2,   Mp * kNQ * 2,  Mp * kFFN * 2,
                                   Mp * 768 * 2, M * kNQ * 2,    M * kNKV * 2,  M * kNKV * 2,
                                   M * (kHD / 2) * sizeof(float2), M * kAD * 4};
  return ws_align256(sz[i]);
}
constexpr size_t call_ws_bytes(int max_batch) {
  size_t n = 0;
  for (int i = 0; i < kCallWsParts; ++i) n += call_ws_part(max_batch, i);
  return n;
}
// Carve a CallWs for max_batch queries from base (call_ws_bytes(max_batch) bytes).
inline CallWs carve_call_ws(char* base, int max_batch) {
  char* p[kCallWsParts];
  size_t off = 0;
  for (int i = 0; i < kCallWsParts; ++i) {
    p[i] = base + off;
    off += call_ws_part(max_batch, i);
  }
  CallWs w;
  w.x = (float*)p[0]; w.h = (float*)p[1];
  w.s16 = (half_t*)p[2]; w.o16 = (half_t*)p[3]; w.u16 = (half_t*)p[4]; w.h16 = (half_t*)p[5];
  w.q = (bf16_t*)p[6]; w.kc = (bf16_t*)p[7]; w.vc = (bf16_t*)p[8];
  w.ropeq = (float2*)p[9];
  w.x2 = (float*)p[10];
  return w;
}

// The no-alloc denoise (smolexp_denoise_noalloc) keeps its per-call workspace in a fixed
// device array of the library, sized for this many queries.
constexpr int kNoAllocMaxBatch = 16;
// Address of that array on `device` (which must be current), looked up once per device;
// nullptr with an error if the lookup failed.
hipError_t noalloc_scratch(int device, char** ptr, size_t* bytes);
// Zero columns 720..767 of rows 0 .. rows-1 (rows a multiple of 16) of an h16 buffer.
hipError_t launch_zero_h16_pad(half_t* h16, int rows, hipStream_t s);

// How one GEMM is cut up (kernels.hip decides, the host sizes workspaces from it).
struct GemmPlan {
  int kind;      // 0: register-resident K split (skinny): 16 rb x 16 cb tiles, 8 waves split K;
                 // 1: register-staged tiles (64 or 128 x 128); 2: pipelined LDS-DMA GEMM
  int kpw;       // skinny: 32-wide k-steps per wave (8 waves)
  int bm;        // tiled: rows per tile (64 or 128)
  int rb;        // skinny: 16-row blocks per workgroup (4, 2 or 1: the rows split over 4 / rb workgroups)
  int cb;        // skinny: 16-column blocks per workgroup (1, 2 or 4)
  int stages;    // pipelined: LDS ring depth (2 or 4); bm = tile rows (64 or 128)
  int ntiles_n;  // output tiles (workgroups) along N
  int reg;       // pipelined: 1 = epilogue from the accumulators (weight fragment as the first MFMA operand)
  int fmw;       // pipelined: 16-row fragments per wave along M (2; 1 = eight waves on 64-row tiles)
};
GemmPlan plan_gemm(int M, int N, int K);

// Large-M GEMM with an LDS-DMA ring (fp16 A, K % 64 == 0): E_QKV and E_SWIGLU on the
// RMSNorm'd residual (norm = true: A = h16), E_H_RESID on a plain fp16 operand.
hipError_t launch_gemm_big(const GemmPlan& p, EMode em, bool norm, const GemmArgs& a, hipStream_t s);
// The kernel and tiles for one projection of the loop (K = logical width).  kind 2 = the
// pipelined GEMM, which reads RMSNorm'd operands over K = kKPad stored columns.
// w8: the weights are E4M3 codes, which only the register-resident kernels read (rb, cb <= 2).
GemmPlan plan_for(int M, int N, int K, AMode am, EMode em, bool w8 = false);
constexpr int kKPad = 768;  // stored columns of h16 and of the weights that read it (a multiple of 64)

// Launchers (kernels.hip).  Each returns the hipGetLastError() after launch.
hipError_t launch_gemm(const GemmPlan& p, AMode am, EMode em, const GemmArgs& a, hipStream_t s);
// The step boundary in one launch (query groups whose action_out takes the register-resident K
// split, up to 4800 rows): v = action_out's arguments (A = fp16(h), lda = 768; no final
// output; the state of step k is read from v.x), t = the next step's time_in arguments (the
// state of step k + 1 is written to t.x, which must be another buffer).  o: the time MLP's
// second layer too (its arguments; groups of at most kBoundaryTimeOutMaxRows rows), or nullptr.
constexpr int kBoundaryTimeOutMaxRows = 64;
hipError_t launch_step_boundary(const GemmArgs& v, const GemmArgs& t, const GemmArgs* o, hipStream_t s);
hipError_t launch_attention(bool self_layer, const AttnArgs& a, hipStream_t s);
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);
hipError_t launch_rope_table(float2* tab, int n_pos, float theta, hipStream_t s);
hipError_t launch_inv_period_table(double* tab, float p_min, float p_max, hipStream_t s);

// Prefill of the prefix language model.
struct PrefillPrologueArgs {
  int* status;             // cleared to 0, then kRangeResidual if an embedding is beyond fp16's range
  int B, P;
  const bf16_t* emb;       // [B][P][960] token embeddings
  const uint8_t* mask;     // [B][P]
  const float2* rope;      // [pos][32] (cos, sin) by position
  float* h;                // out: fp32 residual [B*P][960], blocked (t32_off)
  half_t* h16;             // out: its fp16 copy [B*P][960], blocked (t16_off)
  float2* ropeq;           // out [B*P][32]: the rope rows at each token's position (valid tokens before it)
};
hipError_t launch_prefill_prologue(const PrefillPrologueArgs& a, hipStream_t s);
// Prefix self-attention of a prefill: seq = P query rows per head, keys = the valid prefix tokens.
hipError_t launch_prefix_attention(const AttnArgs& a, hipStream_t s);
// The prefill's projections (M = B*P rows): skinny or pipelined kernels by size.
GemmPlan plan_prefill(int M, int N, int K, EMode em);

}  // namespace smolexp
