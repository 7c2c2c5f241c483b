// Internal interface of the training step (train.hip): argument blocks, workspace layout and
// manifest offsets.  Not part of the C ABI.
#pragma once

#include "smolexp_internal.h"

namespace smolexp {

// C[m][n] = alpha sum_k A(m,k) B(n,k) (+ Cin[m][n], leading dimension ldc) (+ bias[n])
struct TrGemm {
  int M, N, K;
  const void* A;
  int lda;
  const void* B;
  int ldb;
  float* C;
  int ldc;
  const float* Cin;
  const float* bias;
  float alpha;
  float* part;        // k-split scratch (NULL: no split)
  size_t part_cap;    // its capacity in floats
};

struct TrAttn {
  const float* qkv;     // [M][ldq]: Q heads at 64 h, self layers' K at 960 + 64 g, V at 1280 + 64 g (rotated Q, K)
  int ldq;
  const bf16_t* pk;     // this layer's prefix K / V [B][5][P][64]
  const bf16_t* pv;
  const int* vidx;      // [B][P] valid prefix positions, compacted
  const int* nval;      // [B]
  int P;
  float* o;             // [M][960] attention output (forward), read by the backward
  bf16_t* o16;          // forward: the same output in bf16 (the o projection's operand)
  float* lse;           // [B][15][50] log-sum-exp of each score row (INFINITY: no key)
  const float* dout;    // backward: dO [M][960]
  float* dq;            // backward: dQ [M][ldq] at 64 h (rotated space)
  float* dkv;           // backward, self layers: [B][15][2][50][64] per-head dK, dV of the chunk keys
};

struct TrLayerOffsets {
  size_t norm1, qkv, o, norm2, gu, down;
};
struct TrOffsets {
  size_t ain_w, ain_b, tin_w, tin_b, tout_w, tout_b, fnorm, aout_w, aout_b;
  TrLayerOffsets layer;  // of the layer asked for
};
size_t train_offsets(int L, int layer, TrOffsets* o);  // returns the manifest's element count
size_t train_manifest_count(int L);

// Activations kept for the backward pass (fp32, [rows][columns], rows = 50 B) and its scratch.
struct TrainWs {
  float *xt, *target, *z, *s;
  bf16_t* sil;              // SiLU of the time MLP's first layer (an operand only: bf16)
  float *H;                 // [L + 1][M][720] layer inputs (H[0] = time MLP output), H[L] the last output
  float *R1, *QKV, *O, *LSE, *HM, *R2, *GU;  // per layer
  bf16_t *N1, *N2, *ACT, *O16;  // per layer, matrix-product operands only: stored as the bf16 the products read
  bf16_t* NF;
  float *RF, *V;
  float *dv, *dh, *dn, *dact, *dout, *dqkv, *dkv, *part;
  bf16_t *dh16, *dgu;       // bf16 copy of dh, and the SwiGLU gradient (matrix-product operands only)
  bf16_t* dqkv16;           // the Q/K/V gradient after the rotation's transpose, bf16 (a product operand)
  float *split;             // k-split partial sums of the matrix products
  float *split2;            // the same for the products on the side stream
  int *vidx, *nval;
};
size_t train_workspace_bytes(int B, int P, int L);
size_t train_split_cap(int B);  // floats of TrainWs::split
size_t train_carve(char* base, int B, int P, int L, TrainWs* w);  // base NULL: sizes only

struct TrainArgs {
  int B, P, L;
  const bf16_t* kv;        // prefix cache [L][2][B][5][P][64]
  const uint8_t* mask;     // [B][P]
  const float* actions;    // [B][50][32]
  const float* noise;      // [B][50][32]
  const float* t;          // [B]
  float* grads;            // [manifest count] fp32, overwritten
  float* loss;             // [1]
  const bf16_t* w;         // the manifest as loaded, bf16
  const float* bias32;     // fp32 copies of b_in, b_t1, b_t2 (720 each), b_out (32)
  const float2* rope;      // [pos][32] (cos, sin)
  const double* inv_period;  // [360]
  float rms_eps;
  size_t split_cap;        // floats of ws.split and ws.split2 (the workspace's batch)
  hipStream_t side;        // second stream for the layers' weight gradients (default priority)
  hipEvent_t* ev;          // events for its forks and joins, n_ev of them (4 pairs per layer)
  int n_ev;
  TrainWs ws;
};
hipError_t train_enqueue(const TrainArgs& t, hipStream_t s);
hipError_t launch_tr_gemm(const TrGemm& g, bool a_kcont, bool a_bf16, bool b_kcont, bool b_bf16, hipStream_t s);

}  // namespace smolexp
