// The expert's flow-matching training step on gfx950: forward with the activations kept,
// the loss, and the backward pass to every weight gradient.
//
// noeira docs "SmolVLA", Architecture: a training sample is x_t = t eps + (1 - t) a and the
// expert's velocity at (x_t, t) is regressed onto eps - a with a squared error; Fine-tuning:
// only the expert trains, so the prefix keys/values are frozen inputs.  The loss is the mean
// over the batch's B x 50 x 32 elements.
//
// Data layout: activations are row-major [rows][columns] with rows = query * 50 + chunk row,
// fp32 where an elementwise step reads them (residual stream, norms, SwiGLU inputs,
// attention output) and bf16 where only matrix products do (norm outputs, SwiGLU output,
// the gradients that feed products: rounding them when written gives the bits the product
// would form).  The weights are the manifest's bf16 matrices as given ([out][in] row-major);
// the gradients are fp32 in manifest order.  All matrix products run on one bf16 MFMA
// kernel (fp32 accumulate) that reads either operand along or across its contraction axis,
// so the forward (x W^T), the input gradient (dy W) and the weight gradient (dy^T x) need
// no transposed copies.  Attention recomputes its scores in the backward pass from the
// saved log-sum-exp; the prefix keys of a query are read through a compacted list of its
// valid positions, so pads are never touched.
#include "smolexp_internal.h"
#include "smolexp_train.h"

#include <algorithm>

namespace smolexp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t bf16_bits(float f) {  // round to nearest, ties to even (finite inputs)
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

// four consecutive operand values as four bf16 (two per 32-bit word, low half first)
__device__ inline uint2 load4(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return make_uint2(bf16_bits(v.x) | (bf16_bits(v.y) << 16), bf16_bits(v.z) | (bf16_bits(v.w) << 16));
}
__device__ inline uint2 load4(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// ------------------------------------------------------------------------------------------
// C[m][n] = alpha sum_k A(m,k) B(n,k) (+ Cin[m][n]) (+ bias[n])
//   A(m,k) = A[m lda + k] (AK) or A[k lda + m];  B(n,k) = B[n ldb + k] (BK) or B[k ldb + n].
// 128 x 128 tiles, 64-deep k-slabs staged through LDS as bf16 rows of 64 (+ 8 pad), four
// waves of 64 x 64 (4 x 4 MFMA 16x16x32 tiles, two k-steps per slab).  An operand stored
// along k moves in 4-wide vectors; one stored across k is read 4 rows at a time (each load
// coalesced across the lanes) and transposed in registers, so every LDS write is 8 bytes
// either way.  The next slab's loads are issued before the current
// slab's MFMAs.  Out-of-range rows and k read as zero.  With a k-split (gridDim > tiles)
// workgroup group s covers k-slabs [s kc, (s + 1) kc) and writes raw partial sums to
// part[s][M][N]; tr_split_sum_kernel finishes them.
constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;

// LDS element offset of (row r, k) in a slab: the 16-byte chunks of a row are permuted by
// the row's group of 16 (chunk ^ (r / 16) % 8).  The transposed stores write rows 8 apart,
// which with the 144-byte row stride land on only two bank groups unpermuted; with the
// permutation the 16 rows of one store spread over all 64 banks.  The operand reads take
// 16 consecutive rows, one permutation, so they keep the stride's conflict-free pattern.
__device__ inline int slab_off(int r, int k) { return r * GLD + ((((k >> 3) ^ (r >> 4)) & 7) << 3) + (k & 7); }

// four consecutive fp32 values of one row
__device__ inline float4 row4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// One operand's share of a slab, as NV x 4 bf16 per thread.  Stored along k (KC): 4-wide
// vectors of one row.  Stored across k: 4 x 4 blocks (4 k-rows of 4 consecutive operand
// rows, each a 16-byte load coalesced across the lanes), transposed in registers into 4
// rows of 4 k-values; thread t takes operand rows 4 (t % 32) .. +3 and k-quads t / 32 + 8 q.
// R (the operand's row count) is a multiple of 4 there.
constexpr int NV = GBM * GBK / 4 / 256;  // 4-wide vectors per thread per operand and slab

template <typename T, bool KC>
__device__ inline void load_slab(const T* X, int ld, int r0, int R, int k0, int K, int tid, uint2 (&v)[NV]) {
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + 256 * i, r = r0 + idx / (GBK / 4), k = k0 + (idx % (GBK / 4)) * 4;
      v[i] = (r < R && k < K) ? load4(X + (size_t)r * ld + k) : make_uint2(0, 0);
    }
  } else if constexpr (sizeof(T) == 2) {
    // bf16 across k: 4 k-rows x 8 operand rows per thread (16-byte loads), rows 8 (t % 16)
    // .. +7, k-quad t / 16; R is a multiple of 8 here
    static_assert(GBK == 64 && NV == 8, "one 4 x 8 block per thread covers the slab");
    const int r = r0 + (tid & 15) * 8, kb = k0 + (tid >> 4) * 4;
    uint4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = (r < R && kb + u < K) ? *reinterpret_cast<const uint4*>(X + (size_t)(kb + u) * ld + r) : make_uint4(0, 0, 0, 0);
    auto h = [&](const uint4& q, int c) -> uint32_t {  // bf16 c of the 8 in q
      const uint32_t word = (c >> 1) == 0 ? q.x : (c >> 1) == 1 ? q.y : (c >> 1) == 2 ? q.z : q.w;
      return (c & 1) ? (word >> 16) : (word & 0xFFFF);
    };
#pragma unroll
    for (int c = 0; c < 8; ++c)
      v[c] = make_uint2(h(x[0], c) | (h(x[1], c) << 16), h(x[2], c) | (h(x[3], c) << 16));
  } else {
    const int r = r0 + (tid & 31) * 4;
#pragma unroll
    for (int blk = 0; blk < NV / 4; ++blk) {
      const int kb = k0 + (tid >> 5) * 4 + blk * 32;
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = (r < R && kb + u < K) ? row4(X + (size_t)(kb + u) * ld + r) : make_float4(0.f, 0.f, 0.f, 0.f);
      v[blk * 4 + 0] = make_uint2(bf16_bits(x[0].x) | (bf16_bits(x[1].x) << 16), bf16_bits(x[2].x) | (bf16_bits(x[3].x) << 16));
      v[blk * 4 + 1] = make_uint2(bf16_bits(x[0].y) | (bf16_bits(x[1].y) << 16), bf16_bits(x[2].y) | (bf16_bits(x[3].y) << 16));
      v[blk * 4 + 2] = make_uint2(bf16_bits(x[0].z) | (bf16_bits(x[1].z) << 16), bf16_bits(x[2].z) | (bf16_bits(x[3].z) << 16));
      v[blk * 4 + 3] = make_uint2(bf16_bits(x[0].w) | (bf16_bits(x[1].w) << 16), bf16_bits(x[2].w) | (bf16_bits(x[3].w) << 16));
    }
  }
}

template <bool KC, bool H8>
__device__ inline void store_slab(uint16_t* s, int tid, const uint2 (&v)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int r, k;
    if constexpr (KC) {
      const int idx = tid + 256 * i;
      r = idx / (GBK / 4);
      k = (idx % (GBK / 4)) * 4;
    } else if constexpr (H8) {
      r = (tid & 15) * 8 + i;
      k = (tid >> 4) * 4;
    } else {
      r = (tid & 31) * 4 + (i & 3);
      k = (tid >> 5) * 4 + (i >> 2) * 32;
    }
    *reinterpret_cast<uint2*>(s + slab_off(r, k)) = v[i];
  }
}

template <typename TA, bool AK, typename TB, bool BK>
__global__ __launch_bounds__(256) void tr_gemm_kernel(const TrGemm g, int splits, int kc, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[GBM * GLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[GBN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int M = g.M, N = g.N;
  // tiles of one column stripe go to one XCD (workgroup i runs on XCD i % 8), so the
  // B stripe they share is read into one L2
  const int nN = (N + GBN - 1) / GBN, nM = (M + GBM - 1) / GBM, T = nM * nN, per = (T + 7) >> 3;
  const int sidx = (int)blockIdx.x / (8 * per), bid = (int)blockIdx.x % (8 * per);
  const int tile = (bid & 7) * per + (bid >> 3);
  if (tile >= T) return;
  const int n0 = (tile / nM) * GBN, m0 = (tile % nM) * GBM;
  const int kbeg = sidx * kc, kend = min(g.K, kbeg + kc);
  const TA* A = static_cast<const TA*>(g.A);
  const TB* Bm = static_cast<const TB*>(g.B);
  uint2 ra[NV], rb[NV];
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_slab<TA, AK>(A, g.lda, m0, M, kbeg, kend, tid, ra);
  load_slab<TB, BK>(Bm, g.ldb, n0, N, kbeg, kend, tid, rb);
  for (int k0 = kbeg; k0 < kend; k0 += GBK) {
    __syncthreads();  // every wave is done reading the previous slab
    store_slab<AK, sizeof(TA) == 2>(sA, tid, ra);
    store_slab<BK, sizeof(TB) == 2>(sB, tid, rb);
    __syncthreads();
    if (k0 + GBK < kend) {
      load_slab<TA, AK>(A, g.lda, m0, M, k0 + GBK, kend, tid, ra);
      load_slab<TB, BK>(Bm, g.ldb, n0, N, k0 + GBK, kend, tid, rb);
    }
#pragma unroll
    for (int ks = 0; ks < GBK / 32; ++ks) {
      bf16x8 af[4], bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(sA + slab_off(wm * 64 + i * 16 + (lane & 15), ks * 32 + (lane >> 4) * 8));
        bw[i] = *reinterpret_cast<const bf16x8*>(sB + slab_off(wn * 64 + i * 16 + (lane & 15), ks * 32 + (lane >> 4) * 8));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
  }
  // lane l of a 16 x 16 tile holds rows 4 (l / 16) + r, column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r, col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (row < M && col < N) {
          if (splits > 1) {
            part[((size_t)sidx * M + row) * N + col] = acc[i][j][r];
          } else {
            float v = g.alpha * acc[i][j][r];
            if (g.Cin) v += g.Cin[(size_t)row * g.ldc + col];
            if (g.bias) v += g.bias[col];
            g.C[(size_t)row * g.ldc + col] = v;
          }
        }
      }
}

// C[m][n] = alpha sum_s part[s][m][n] (+ Cin) (+ bias), the parts added in order; four
// columns per thread (N and ldc are multiples of 4).
__global__ __launch_bounds__(256) void tr_split_sum_kernel(const TrGemm g, int splits, const float* part) {
  const int n4 = g.N >> 2, total = g.M * n4;
  const size_t stride = (size_t)g.M * g.N;
  for (int q = blockIdx.x * 256 + threadIdx.x; q < total; q += gridDim.x * 256) {
    const int row = q / n4, c = (q - row * n4) * 4;
    const size_t e = (size_t)row * g.N + c;
    float4 v = *reinterpret_cast<const float4*>(part + e);
    for (int s = 1; s < splits; ++s) {
      const float4 x = *reinterpret_cast<const float4*>(part + (size_t)s * stride + e);
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    v.x *= g.alpha; v.y *= g.alpha; v.z *= g.alpha; v.w *= g.alpha;
    const size_t o = (size_t)row * g.ldc + c;
    if (g.Cin) {
      const float4 x = *reinterpret_cast<const float4*>(g.Cin + o);
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    if (g.bias) {
      const float4 x = *reinterpret_cast<const float4*>(g.bias + c);
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    *reinterpret_cast<float4*>(g.C + o) = v;
  }
}

// ------------------------------------------------------------------------------------------
// Per query: the compacted list of valid prefix positions and their count.
__global__ __launch_bounds__(64) void tr_prep_kernel(const uint8_t* mask, int P, int* vidx, int* nval) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int n = 0;
  for (int j0 = 0; j0 < P; j0 += 64) {
    const int j = j0 + lane;
    const bool v = j < P && mask[(size_t)b * P + j] != 0;
    const uint64_t bal = __ballot(v);
    if (v) vidx[(size_t)b * P + n + __popcll(bal & ((1ull << lane) - 1))] = j;
    n += __popcll(bal);
  }
  if (lane == 0) nval[b] = n;
}

// Training inputs of one chunk row: x_t = t eps + (1 - t) a, the target eps - a, and the
// time embedding e(t) of the row's query in columns 720.. of z (z = [action_in(x_t) ; e(t)]).
__global__ __launch_bounds__(256) void tr_input_kernel(const float* act, const float* noise, const float* t,
                                                       const double* inv_period, float* xt, float* target, float* z) {
  const int row = blockIdx.x, b = row / kChunk, tid = threadIdx.x;
  const float tb = t[b];
  if (tid < kAD) {
    const size_t o = (size_t)row * kAD + tid;
    const float e = noise[o], a = act[o];
    xt[o] = tb * e + (1.f - tb) * a;
    target[o] = e - a;
  }
  for (int k = tid; k < kD; k += 256) {
    const int half = kD / 2, kk = k % half;
    const double ang = 6.283185307179586 * (double)tb * inv_period[kk];
    z[(size_t)row * (2 * kD) + kD + k] = (float)(k < half ? sin(ang) : cos(ang));
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// RMSNorm of 720-wide rows, one wave per row: n = h r g with r = (mean(h^2) + eps)^(-1/2).
__global__ __launch_bounds__(256) void tr_rmsnorm_kernel(const float* h, const bf16_t* g, float eps, int M, bf16_t* n,
                                                         float* rstd) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  constexpr int Q = kD / 4;  // 180 column quads; lane takes quads lane, lane + 64, lane + 128
  const float4* hr = reinterpret_cast<const float4*>(h + (size_t)row * kD);
  float4 x[3];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int c4 = lane + 64 * u;
    x[u] = c4 < Q ? hr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += x[u].x * x[u].x + x[u].y * x[u].y + x[u].z * x[u].z + x[u].w * x[u].w;
  }
  const float r = rsqrtf(wave_sum(ss) / kD + eps);
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int c4 = lane + 64 * u;
    if (c4 < Q) {
      const uint2 gg = *reinterpret_cast<const uint2*>(g + 4 * c4);
      *reinterpret_cast<uint2*>(n + (size_t)row * kD + 4 * c4) =
          make_uint2(bf16_bits(x[u].x * r * bf16_val(gg.x & 0xFFFF)) | (bf16_bits(x[u].y * r * bf16_val(gg.x >> 16)) << 16),
                     bf16_bits(x[u].z * r * bf16_val(gg.y & 0xFFFF)) | (bf16_bits(x[u].w * r * bf16_val(gg.y >> 16)) << 16));
    }
  }
  if (lane == 0) rstd[row] = r;
}

// Backward of the RMSNorm above over kRB rows per workgroup:
//   dh = r (u - hat mean(u hat)) (+ resid), u = dy g, hat = h r;
//   part[blk][c] = sum over the block's rows of dy hat (the gain's gradient, before the
//   sum over blocks).  dh may alias resid; dh16 receives dh in bf16 (a product operand).
//   Phase 1: each wave forms mean(u hat) of its rows (4-wide loads); phase 2: thread t
//   takes columns 4t .. 4t + 3 of all kRB rows (the second
//   read of dy and h comes from L2).
constexpr int kRB = 8;
__global__ __launch_bounds__(256) void tr_rmsnorm_bwd_kernel(const float* dy, const float* h, const float* rstd,
                                                             const bf16_t* g, const float* resid, float* dh,
                                                             bf16_t* dh16, int M, float* part) {
  __shared__ float smean[kRB];
  const int blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int Q = kD / 4;  // 180 column quads
  for (int rr = w; rr < kRB; rr += 4) {
    const int row = blk * kRB + rr;
    float s = 0.f;
    if (row < M) {
      const float r = rstd[row];
      for (int c4 = lane; c4 < Q; c4 += 64) {
        const float4 d = *reinterpret_cast<const float4*>(dy + (size_t)row * kD + 4 * c4);
        const float4 x = *reinterpret_cast<const float4*>(h + (size_t)row * kD + 4 * c4);
        const uint2 gg = *reinterpret_cast<const uint2*>(g + 4 * c4);
        s += d.x * bf16_val(gg.x & 0xFFFF) * x.x + d.y * bf16_val(gg.x >> 16) * x.y +
             d.z * bf16_val(gg.y & 0xFFFF) * x.z + d.w * bf16_val(gg.y >> 16) * x.w;
      }
      s = wave_sum(s) * r / kD;
    }
    if (lane == 0) smean[rr] = s;
  }
  __syncthreads();
  if (tid < Q) {
    const uint2 gg = *reinterpret_cast<const uint2*>(g + 4 * tid);
    const float g0 = bf16_val(gg.x & 0xFFFF), g1 = bf16_val(gg.x >> 16), g2 = bf16_val(gg.y & 0xFFFF),
                g3 = bf16_val(gg.y >> 16);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int rr = 0; rr < kRB; ++rr) {
      const int row = blk * kRB + rr;
      if (row >= M) break;
      const float r = rstd[row], mean = smean[rr];
      const size_t o = (size_t)row * kD + 4 * tid;
      const float4 d = *reinterpret_cast<const float4*>(dy + o);
      const float4 x = *reinterpret_cast<const float4*>(h + o);
      float4 v;
      v.x = r * (d.x * g0 - x.x * r * mean);
      v.y = r * (d.y * g1 - x.y * r * mean);
      v.z = r * (d.z * g2 - x.z * r * mean);
      v.w = r * (d.w * g3 - x.w * r * mean);
      if (resid) {
        const float4 q = *reinterpret_cast<const float4*>(resid + o);
        v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
      }
      *reinterpret_cast<float4*>(dh + o) = v;
      *reinterpret_cast<uint2*>(dh16 + o) =
          make_uint2(bf16_bits(v.x) | (bf16_bits(v.y) << 16), bf16_bits(v.z) | (bf16_bits(v.w) << 16));
      acc.x += d.x * x.x * r;
      acc.y += d.y * x.y * r;
      acc.z += d.z * x.z * r;
      acc.w += d.w * x.w * r;
    }
    *reinterpret_cast<float4*>(part + (size_t)blk * kD + 4 * tid) = acc;
  }
}

// Column sums of x [M][N] over blocks of kRB rows: part[blk][c].
__global__ __launch_bounds__(256) void tr_colsum_kernel(const float* x, int M, int N, float* part) {
  const int c = blockIdx.x * 256 + threadIdx.x, blk = blockIdx.y;
  if (c >= N) return;
  float s = 0.f;
  for (int rr = 0; rr < kRB; ++rr) {
    const int row = blk * kRB + rr;
    if (row >= M) break;
    s += x[(size_t)row * N + c];
  }
  part[(size_t)blk * N + c] = s;
}

// out[c] = sum over blocks of part[blk][c]: 16 columns per workgroup, thread group u of 16
// adds the blocks blk = u mod 16 in order, and the 16 sums are added in group order
// (deterministic).
__global__ __launch_bounds__(256) void tr_reduce_kernel(const float* part, int nblk, int N, float* out) {
  __shared__ float red[16][17];
  const int cl = threadIdx.x & 15, u = threadIdx.x >> 4, c = blockIdx.x * 16 + cl;
  float s = 0.f;
  if (c < N)
    for (int b = u; b < nblk; b += 16) s += part[(size_t)b * N + c];
  red[u][cl] = s;
  __syncthreads();
  if (u == 0 && c < N) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][cl];
    out[c] = t;
  }
}

__device__ inline float silu_f(float z) { return z / (1.f + __expf(-z)); }
__device__ inline float silu_grad_f(float z) {
  const float s = 1.f / (1.f + __expf(-z));
  return s * (1.f + z * (1.f - s));
}

__global__ __launch_bounds__(256) void tr_silu_kernel(const float* s, bf16_t* out, size_t n) {
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) out[i] = (bf16_t)bf16_bits(silu_f(s[i]));
}
__global__ __launch_bounds__(256) void tr_silu_bwd_kernel(const float* d, const float* s, float* out, size_t n) {
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) out[i] = d[i] * silu_grad_f(s[i]);
}

// gu [M][4096] = [gate | up]; act = SiLU(gate) up.  Four columns per thread.
__global__ __launch_bounds__(256) void tr_swiglu_kernel(const float* gu, bf16_t* act, size_t n) {
  for (size_t q = blockIdx.x * 256 + threadIdx.x; q < n / 4; q += (size_t)gridDim.x * 256) {
    const size_t row = q / (kFFN / 4), c = (q % (kFFN / 4)) * 4;
    const float4 gt = *reinterpret_cast<const float4*>(gu + row * kGU + c);
    const float4 up = *reinterpret_cast<const float4*>(gu + row * kGU + kFFN + c);
    *reinterpret_cast<uint2*>(act + row * kFFN + c) =
        make_uint2(bf16_bits(silu_f(gt.x) * up.x) | (bf16_bits(silu_f(gt.y) * up.y) << 16),
                   bf16_bits(silu_f(gt.z) * up.z) | (bf16_bits(silu_f(gt.w) * up.w) << 16));
  }
}
__global__ __launch_bounds__(256) void tr_swiglu_bwd_kernel(const float* dact, const float* gu, bf16_t* dgu, size_t n) {
  for (size_t q = blockIdx.x * 256 + threadIdx.x; q < n / 4; q += (size_t)gridDim.x * 256) {
    const size_t row = q / (kFFN / 4), c = (q % (kFFN / 4)) * 4;
    const float4 gt = *reinterpret_cast<const float4*>(gu + row * kGU + c);
    const float4 up = *reinterpret_cast<const float4*>(gu + row * kGU + kFFN + c);
    const float4 d = *reinterpret_cast<const float4*>(dact + row * kFFN + c);
    *reinterpret_cast<uint2*>(dgu + row * kGU + c) =
        make_uint2(bf16_bits(d.x * up.x * silu_grad_f(gt.x)) | (bf16_bits(d.y * up.y * silu_grad_f(gt.y)) << 16),
                   bf16_bits(d.z * up.z * silu_grad_f(gt.z)) | (bf16_bits(d.w * up.w * silu_grad_f(gt.w)) << 16));
    *reinterpret_cast<uint2*>(dgu + row * kGU + kFFN + c) =
        make_uint2(bf16_bits(d.x * silu_f(gt.x)) | (bf16_bits(d.y * silu_f(gt.y)) << 16),
                   bf16_bits(d.z * silu_f(gt.z)) | (bf16_bits(d.w * silu_f(gt.w)) << 16));
  }
}

// RoPE (pairs d, d + 32) on the Q heads (and the self layers' K heads) of qkv rows, in place,
// at position n_valid(b) + i.  dir = +1 rotates, -1 applies the transpose (the backward);
// out16 non-NULL: the result goes there in bf16 instead of back into qkv.
__global__ __launch_bounds__(256) void tr_rope_kernel(float* qkv, int ldq, int n_heads, const int* nval,
                                                      const float2* rope, float dir, bf16_t* out16) {
  const int row = blockIdx.x, b = row / kChunk, i = row % kChunk;
  const float2* cs = rope + (size_t)(nval[b] + i) * (kHD / 2);
  for (int p = threadIdx.x; p < n_heads * (kHD / 2); p += 256) {
    const int hd = p / (kHD / 2), k = p % (kHD / 2);
    float* x = qkv + (size_t)row * ldq + hd * kHD;
    const float c = cs[k].x, s = dir * cs[k].y;
    const float x1 = x[k], x2 = x[k + kHD / 2], y1 = x1 * c - x2 * s, y2 = x1 * s + x2 * c;
    if (out16) {  // the backward: the rotated gradient goes to its bf16 copy (a product operand)
      bf16_t* y = out16 + (size_t)row * ldq + hd * kHD;
      y[k] = (bf16_t)bf16_bits(y1);
      y[k + kHD / 2] = (bf16_t)bf16_bits(y2);
    } else {
      x[k] = y1;
      x[k + kHD / 2] = y2;
    }
  }
}

// Self layers: the chunk keys' gradients, summed over the three query heads of each KV head
// from the per-head parts dkv [B][15][2][50][64], into columns 960.. (K, rotated back) and
// 1280.. (V) of dqkv's bf16 copy.
__global__ __launch_bounds__(256) void tr_kv_grad_kernel(const float* dkv, const int* nval, const float2* rope,
                                                         bf16_t* dqkv) {
  const int row = blockIdx.x, b = row / kChunk, i = row % kChunk;
  const float2* cs = rope + (size_t)(nval[b] + i) * (kHD / 2);
  auto part = [&](int h, int kv, int d) {
    return dkv[((((size_t)b * kHQ + h) * 2 + kv) * kChunk + i) * kHD + d];
  };
  const int grp = kHQ / kHKV;
  for (int p = threadIdx.x; p < kHKV * (kHD / 2); p += 256) {
    const int g = p / (kHD / 2), k = p % (kHD / 2);
    float y1 = 0.f, y2 = 0.f;
    for (int u = 0; u < grp; ++u) {
      y1 += part(g * grp + u, 0, k);
      y2 += part(g * grp + u, 0, k + kHD / 2);
    }
    const float c = cs[k].x, s = cs[k].y;
    bf16_t* x = dqkv + (size_t)row * kNQKV + kNQ + g * kHD;
    x[k] = (bf16_t)bf16_bits(y1 * c + y2 * s);
    x[k + kHD / 2] = (bf16_t)bf16_bits(-y1 * s + y2 * c);
  }
  for (int p = threadIdx.x; p < kNKV; p += 256) {
    const int g = p / kHD, d = p % kHD;
    float y = 0.f;
    for (int u = 0; u < grp; ++u) y += part(g * grp + u, 1, d);
    dqkv[(size_t)row * kNQKV + kNQ + kNKV + p] = (bf16_t)bf16_bits(y);
  }
}

// Loss terms over 8 rows per workgroup: err = v - target, dv = 2 err / n_total, and the
// block's sum of err^2.
__global__ __launch_bounds__(256) void tr_loss_kernel(const float* v, const float* target, int M, float inv_n,
                                                      float* dv, float* part) {
  __shared__ float red[4];
  const int row = blockIdx.x * 8 + (threadIdx.x >> 5), c = threadIdx.x & 31;
  float e2 = 0.f;
  if (row < M) {
    const size_t o = (size_t)row * kAD + c;
    const float err = v[o] - target[o];
    dv[o] = 2.f * err * inv_n;
    e2 = err * err;
  }
  e2 = wave_sum(e2);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = e2;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void tr_scale_kernel(float* x, float s) { *x *= s; }

// ------------------------------------------------------------------------------------------
// Attention of one (query, Q head) per workgroup over its keys: the valid prefix keys (from
// the compacted position list), then, in self layers, the chunk's keys j <= i.  Four waves
// of 16 query rows (rows 50..63 are padding).  Scores and products run on bf16 MFMA
// 16x16x32 with fp32 accumulation: S = Q K^T per 64-key block (Q pre-scaled by 1/8), an
// online softmax in fp32 (running row maximum and sum, kept as the log-sum-exp for the
// backward pass), and O += P V with V transposed in LDS and P passed through a per-wave
// LDS tile from the accumulator layout to the operand layout.
constexpr int kKB = 64;      // keys per block
constexpr int kRows = kChunk;
constexpr int KLD = kHD + 8;  // bf16 row stride of the LDS tiles (144 bytes)

// lane l of an MFMA 16x16 accumulator tile holds rows 4 (l / 16) + r, column l % 16; an
// operand fragment holds row l % 16, k = 8 (l / 16) .. +7
__device__ inline bf16x8 frag_ld(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ inline bf16x8 frag_from_f32(const float* p) {  // 8 consecutive fp32 values -> bf16x8
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  uint4 u;
  u.x = bf16_bits(a.x) | (bf16_bits(a.y) << 16);
  u.y = bf16_bits(a.z) | (bf16_bits(a.w) << 16);
  u.z = bf16_bits(b.x) | (bf16_bits(b.y) << 16);
  u.w = bf16_bits(b.z) | (bf16_bits(b.w) << 16);
  return *reinterpret_cast<const bf16x8*>(&u);
}

// One 64-key block into LDS as bf16: K and V by key ([key][dim]) and, when asked, K or V
// transposed ([dim][key]).  Thread t moves key t / 4, dims 16 (t % 4) .. +15; keys past
// the last one are zero.
template <bool SELF>
__device__ inline void load_block(const TrAttn& a, int b, int g, int nb, int kb, uint16_t* sk, uint16_t* sv,
                                  uint16_t* skt, uint16_t* svt) {
  const int tid = threadIdx.x, j = tid >> 2, d0 = (tid & 3) * 16, kidx = kb * kKB + j;
  uint32_t kk[16], vv[16];
  if (kidx < nb) {
    const size_t o = (((size_t)b * kHKV + g) * a.P + a.vidx[(size_t)b * a.P + kidx]) * kHD + d0;
    const uint4 k0 = *reinterpret_cast<const uint4*>(a.pk + o), k1 = *reinterpret_cast<const uint4*>(a.pk + o + 8);
    const uint4 v0 = *reinterpret_cast<const uint4*>(a.pv + o), v1 = *reinterpret_cast<const uint4*>(a.pv + o + 8);
    const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      kk[2 * u] = kw[u] & 0xFFFF;
      kk[2 * u + 1] = kw[u] >> 16;
      vv[2 * u] = vw[u] & 0xFFFF;
      vv[2 * u + 1] = vw[u] >> 16;
    }
  } else if (SELF && kidx < nb + kChunk) {
    const float* src = a.qkv + (size_t)(b * kChunk + kidx - nb) * a.ldq;
#pragma unroll
    for (int u = 0; u < 16; u += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + kNQ + g * kHD + d0 + u);
      const float4 y = *reinterpret_cast<const float4*>(src + kNQ + kNKV + g * kHD + d0 + u);
      kk[u] = bf16_bits(x.x); kk[u + 1] = bf16_bits(x.y); kk[u + 2] = bf16_bits(x.z); kk[u + 3] = bf16_bits(x.w);
      vv[u] = bf16_bits(y.x); vv[u + 1] = bf16_bits(y.y); vv[u + 2] = bf16_bits(y.z); vv[u + 3] = bf16_bits(y.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) kk[u] = vv[u] = 0u;
  }
#pragma unroll
  for (int u = 0; u < 16; u += 8) {
    uint4 pk, pv;
    pk.x = kk[u] | (kk[u + 1] << 16); pk.y = kk[u + 2] | (kk[u + 3] << 16);
    pk.z = kk[u + 4] | (kk[u + 5] << 16); pk.w = kk[u + 6] | (kk[u + 7] << 16);
    pv.x = vv[u] | (vv[u + 1] << 16); pv.y = vv[u + 2] | (vv[u + 3] << 16);
    pv.z = vv[u + 4] | (vv[u + 5] << 16); pv.w = vv[u + 6] | (vv[u + 7] << 16);
    if (sk) *reinterpret_cast<uint4*>(sk + j * KLD + d0 + u) = pk;
    if (sv) *reinterpret_cast<uint4*>(sv + j * KLD + d0 + u) = pv;
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if (skt) skt[(d0 + u) * KLD + j] = (uint16_t)kk[u];
    if (svt) svt[(d0 + u) * KLD + j] = (uint16_t)vv[u];
  }
}

template <bool SELF>
__device__ inline bool key_ok(int kidx, int nb, int i) {
  return i < kRows && (kidx < nb || (SELF && kidx < nb + kChunk && kidx - nb <= i));
}

// Q (pre-scaled) or dO rows of this wave as the two operand fragments of a 64-deep product.
__device__ inline void row_frags(const float* src, size_t ld, int b, int col0, int w, int lane, float scale,
                                 bf16x8 (&f)[2]) {
  const int i = 16 * w + (lane & 15);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (i < kRows) {
      float x[8];
      const float* p = src + (size_t)(b * kChunk + i) * ld + col0 + ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = p[u] * scale;
      f[ks] = frag_from_f32(x);
    } else {
      f[ks] = bf16x8{};
    }
  }
}

struct AttnSmem {
  uint16_t k[kKB * KLD];
  uint16_t vt[kHD * KLD];
  uint16_t p[4][16 * KLD];
};

template <bool SELF>
__global__ __launch_bounds__(256) void tr_attn_fwd_kernel(const TrAttn a) {
  __shared__ __attribute__((aligned(16))) AttnSmem sm;
  const int h = blockIdx.x, b = blockIdx.y, g = h / (kHQ / kHKV);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q4 = lane >> 4, c16 = lane & 15;
  const int nb = a.nval[b], nk = nb + (SELF ? kChunk : 0), nblk = (nk + kKB - 1) / kKB;
  bf16x8 qf[2];
  row_frags(a.qkv, a.ldq, b, h * kHD, w, lane, 0.125f, qf);
  float m[4], l[4];
  f32x4 o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
    o[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint16_t* sp = sm.p[w];
  for (int kb = 0; kb < nblk; ++kb) {
    __syncthreads();
    load_block<SELF>(a, b, g, nb, kb, sm.k, nullptr, nullptr, sm.vt);
    __syncthreads();
    f32x4 s[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], frag_ld(sm.k + (jt * 16 + c16) * KLD + ks * 32 + q4 * 8),
                                                       s[jt], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * q4 + r;
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (!key_ok<SELF>(kb * kKB + jt * 16 + c16, nb, i)) s[jt][r] = -INFINITY;
        mx = fmaxf(mx, s[jt][r]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m[r], mx);
      const float corr = mn == -INFINITY ? 1.f : __expf(m[r] - mn);
      float sum = 0.f;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const float p = s[jt][r] == -INFINITY ? 0.f : __expf(s[jt][r] - mn);
        sum += p;
        sp[(4 * q4 + r) * KLD + jt * 16 + c16] = (uint16_t)bf16_bits(p);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
      l[r] = l[r] * corr + sum;
      m[r] = mn;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][r] *= corr;
    }
    __syncthreads();  // this wave's P tile is written
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pf = frag_ld(sp + c16 * KLD + ks * 32 + q4 * 8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, frag_ld(sm.vt + (dt * 16 + c16) * KLD + ks * 32 + q4 * 8),
                                                       o[dt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * q4 + r;
    if (i < kRows) {
      const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const size_t e = (size_t)(b * kChunk + i) * kNQ + h * kHD + dt * 16 + c16;
        a.o[e] = o[dt][r] * inv;
        a.o16[e] = (bf16_t)bf16_bits(o[dt][r] * inv);
      }
      if (c16 == 0) a.lse[((size_t)b * kHQ + h) * kRows + i] = l[r] > 0.f ? m[r] + __logf(l[r]) : INFINITY;
    }
  }
}

// Backward of the attention above, one (query, Q head) per workgroup.  D_i = dO_i . O_i;
// per key block: S = Q K^T and dP = dO V^T on MFMA, P = exp(S - lse), dS = P (dP - D);
// dQ += dS K on MFMA (K transposed in LDS); the chunk's keys (self layers) get this head's
// dK = dS^T Q and dV = P^T dO in dkv, on MFMA too (dS, P, Q and dO transposed in LDS).  Q is pre-scaled, so S and dK
// carry the 1/8 already; dQ takes it at the end.
struct AttnBwdSmem {
  uint16_t k[kKB * KLD];
  uint16_t v[kKB * KLD];
  uint16_t kt[kHD * KLD];
  uint16_t ds16[64 * KLD];   // dS by row ([row][key]): the operand of dQ = dS K
  // self layers: the chunk keys' dK = dS^T Q and dV = P^T dO on MFMA need dS and P by key
  // and Q (scaled) and dO by dimension ([.][row], rows 50..63 zero)
  uint16_t dst[kKB * KLD];
  uint16_t pt[kKB * KLD];
  uint16_t qt[kHD * KLD];
  uint16_t dot[kHD * KLD];
  float dd[64], lse[64];
};

template <bool SELF>
__global__ __launch_bounds__(256) void tr_attn_bwd_kernel(const TrAttn a) {
  __shared__ __attribute__((aligned(16))) AttnBwdSmem sm;
  const int h = blockIdx.x, b = blockIdx.y, g = h / (kHQ / kHKV);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q4 = lane >> 4, c16 = lane & 15;
  const int nb = a.nval[b], nk = nb + (SELF ? kChunk : 0), nblk = (nk + kKB - 1) / kKB;
  const float scale = 0.125f;
  if (SELF) {
    for (int e = tid; e < 64 * kHD; e += 256) {
      const int i = e / kHD, d = e % kHD;
      const size_t row = (size_t)(b * kChunk + i);
      sm.qt[d * KLD + i] = i < kRows ? (uint16_t)bf16_bits(a.qkv[row * a.ldq + h * kHD + d] * scale) : 0;
      sm.dot[d * KLD + i] = i < kRows ? (uint16_t)bf16_bits(a.dout[row * kNQ + h * kHD + d]) : 0;
    }
  }
  for (int i = w; i < 64; i += 4) {
    float s = 0.f;
    if (i < kRows) {
      const size_t row = (size_t)(b * kChunk + i);
      s = wave_sum(a.dout[row * kNQ + h * kHD + lane] * a.o[row * kNQ + h * kHD + lane]);
    }
    if (lane == 0) {
      sm.dd[i] = s;
      sm.lse[i] = i < kRows ? a.lse[((size_t)b * kHQ + h) * kRows + i] : INFINITY;
    }
  }
  bf16x8 qf[2], df[2];
  row_frags(a.qkv, a.ldq, b, h * kHD, w, lane, scale, qf);
  row_frags(a.dout, kNQ, b, h * kHD, w, lane, 1.f, df);
  f32x4 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  float lse_r[4], dd_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lse_r[r] = sm.lse[16 * w + 4 * q4 + r];
    dd_r[r] = sm.dd[16 * w + 4 * q4 + r];
  }
  for (int kb = 0; kb < nblk; ++kb) {
    __syncthreads();
    load_block<SELF>(a, b, g, nb, kb, sm.k, sm.v, sm.kt, nullptr);
    __syncthreads();
    f32x4 s[4], dp[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      s[jt] = dp[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off = (jt * 16 + c16) * KLD + ks * 32 + q4 * 8;
        s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], frag_ld(sm.k + off), s[jt], 0, 0, 0);
        dp[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(df[ks], frag_ld(sm.v + off), dp[jt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * q4 + r;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = jt * 16 + c16;
        const float p = key_ok<SELF>(kb * kKB + j, nb, i) ? __expf(s[jt][r] - lse_r[r]) : 0.f;
        const float d = p * (dp[jt][r] - dd_r[r]);
        sm.ds16[i * KLD + j] = (uint16_t)bf16_bits(d);
        if (SELF) {
          sm.pt[j * KLD + i] = (uint16_t)bf16_bits(p);
          sm.dst[j * KLD + i] = (uint16_t)bf16_bits(d);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 dsf = frag_ld(sm.ds16 + (16 * w + c16) * KLD + ks * 32 + q4 * 8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        dq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsf, frag_ld(sm.kt + (dt * 16 + c16) * KLD + ks * 32 + q4 * 8),
                                                        dq[dt], 0, 0, 0);
    }
    if constexpr (SELF) {
      // chunk keys in this block: wave w takes keys 16 w .. 16 w + 15 of it
      const int c0 = kb * kKB + 16 * w - nb;  // chunk index of the wave's first key
      if (c0 + 16 > 0 && c0 < kChunk) {
        f32x4 dk[4], dv[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int off = (16 * w + c16) * KLD + ks * 32 + q4 * 8;
          const bf16x8 dsf = frag_ld(sm.dst + off), pf = frag_ld(sm.pt + off);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int offd = (dt * 16 + c16) * KLD + ks * 32 + q4 * 8;
            dk[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsf, frag_ld(sm.qt + offd), dk[dt], 0, 0, 0);
            dv[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, frag_ld(sm.dot + offd), dv[dt], 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = c0 + 4 * q4 + r;
          if (c >= 0 && c < kChunk) {
            const size_t o = ((((size_t)b * kHQ + h) * 2) * kChunk + c) * kHD + c16;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              a.dkv[o + dt * 16] = dk[dt][r];
              a.dkv[o + (size_t)kChunk * kHD + dt * 16] = dv[dt][r];
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * q4 + r;
    if (i < kRows)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) a.dq[(size_t)(b * kChunk + i) * a.ldq + h * kHD + dt * 16 + c16] = dq[dt][r] * scale;
  }
}

inline int ew_grid(size_t n) { return (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192); }

}  // namespace

// ------------------------------------------------------------------------------------------
hipError_t launch_tr_gemm(const TrGemm& g, bool a_kcont, bool a_bf16, bool b_kcont, bool b_bf16, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  // operands are read in 4-wide vectors along their contiguous axis (K, or the operand's
  // rows M / N when stored across k; 8-wide for bf16 stored across k): that length and the
  // leading dimension must be multiples of the width, so a vector never straddles an edge
  const int wa = (!a_kcont && a_bf16) ? 8 : 4, wb = (!b_kcont && b_bf16) ? 8 : 4;
  if (g.K <= 0 || g.lda % wa || g.ldb % wb || (a_kcont ? g.K : g.M) % wa || (b_kcont ? g.K : g.N) % wb)
    return hipErrorInvalidValue;
  const int T = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN), per = (T + 7) / 8;
  const int nslab = (g.K + GBK - 1) / GBK;
  // k-split: enough workgroups for two per CU, at least 4 slabs each, parts within the scratch
  // (one per CU measured slower: the 128 x 128 tiles are latency-bound at 2 waves per SIMD)
  int splits = 1;
  if (g.part && T < 512) {
    splits = (512 + T - 1) / T;
    splits = min(splits, max(1, nslab / 4));
    while (splits > 1 && (size_t)splits * g.M * g.N > g.part_cap) --splits;
  }
  const int kc = ((nslab + splits - 1) / splits) * GBK;
  splits = (g.K + kc - 1) / kc;
  const dim3 grid(8 * per * splits), block(256);
  if (!a_bf16 && a_kcont && b_bf16 && b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<float, true, bf16_t, true>), grid, block, 0, s, g, splits, kc, g.part);
  else if (!a_bf16 && a_kcont && b_bf16 && !b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<float, true, bf16_t, false>), grid, block, 0, s, g, splits, kc, g.part);
  else if (!a_bf16 && !a_kcont && !b_bf16 && !b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<float, false, float, false>), grid, block, 0, s, g, splits, kc, g.part);
  else if (a_bf16 && a_kcont && b_bf16 && b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<bf16_t, true, bf16_t, true>), grid, block, 0, s, g, splits, kc, g.part);
  else if (!a_bf16 && !a_kcont && b_bf16 && !b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<float, false, bf16_t, false>), grid, block, 0, s, g, splits, kc, g.part);
  else if (a_bf16 && a_kcont && b_bf16 && !b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<bf16_t, true, bf16_t, false>), grid, block, 0, s, g, splits, kc, g.part);
  else if (a_bf16 && !a_kcont && b_bf16 && !b_kcont)
    hipLaunchKernelGGL((tr_gemm_kernel<bf16_t, false, bf16_t, false>), grid, block, 0, s, g, splits, kc, g.part);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const size_t n4 = (size_t)g.M * g.N / 4;
  const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(tr_split_sum_kernel, dim3(blocks), dim3(256), 0, s, g, splits, g.part);
  return hipGetLastError();
}

size_t train_manifest_count(int L) {
  TrOffsets o;
  return train_offsets(L, 0, &o);
}

// Offsets (elements) of every tensor in the weight manifest; returns the total.
size_t train_offsets(int L, int layer, TrOffsets* o) {
  size_t off = 0;
  auto take = [&](size_t n) { size_t v = off; off += n; return v; };
  o->ain_w = take((size_t)kD * kAD);
  o->ain_b = take(kD);
  o->tin_w = take((size_t)kD * 2 * kD);
  o->tin_b = take(kD);
  o->tout_w = take((size_t)kD * kD);
  o->tout_b = take(kD);
  for (int l = 0; l < L; ++l) {
    const bool self = l % 2 == 0;
    TrLayerOffsets lo;
    lo.norm1 = take(kD);
    lo.qkv = take((size_t)(self ? kNQKV : kNQ) * kD);  // q, then k and v: one [1600|960][720] matrix
    lo.o = take((size_t)kD * kNQ);
    lo.norm2 = take(kD);
    lo.gu = take((size_t)kGU * kD);  // gate, then up: one [4096][720] matrix
    lo.down = take((size_t)kD * kFFN);
    if (l == layer) o->layer = lo;
  }
  o->fnorm = take(kD);
  o->aout_w = take((size_t)kAD * kD);
  o->aout_b = take(kAD);
  return off;
}

// k-split partial sums: up to four parts of the largest product output (M x 2048 or 4096 x 720)
size_t train_split_cap(int B) {
  const size_t M = (size_t)B * kChunk;
  return 4 * std::max(M * kFFN, (size_t)kGU * kD);
}

size_t train_workspace_bytes(int B, int P, int L) {
  TrainWs w;
  return train_carve(nullptr, B, P, L, &w);
}

size_t train_carve(char* base, int B, int P, int L, TrainWs* w) {
  const size_t M = (size_t)B * kChunk, nblk = (M + kRB - 1) / kRB;
  size_t off = 0;
  auto f = [&](size_t n) { size_t o = off; off += (n * 4 + 255) & ~(size_t)255; return base ? (float*)(base + o) : nullptr; };
  auto hb = [&](size_t n) { size_t o = off; off += (n * 2 + 255) & ~(size_t)255; return base ? (bf16_t*)(base + o) : nullptr; };
  w->xt = f(M * kAD);
  w->target = f(M * kAD);
  w->z = f(M * 2 * kD);
  w->s = f(M * kD);
  w->sil = hb(M * kD);
  w->H = f((size_t)(L + 1) * M * kD);
  w->N1 = hb((size_t)L * M * kD);
  w->R1 = f((size_t)L * M);
  w->QKV = f((size_t)L * M * kNQKV);
  w->O = f((size_t)L * M * kNQ);
  w->O16 = hb((size_t)L * M * kNQ);
  w->LSE = f((size_t)L * B * kHQ * kChunk);
  w->HM = f((size_t)L * M * kD);
  w->N2 = hb((size_t)L * M * kD);
  w->R2 = f((size_t)L * M);
  w->GU = f((size_t)L * M * kGU);
  w->ACT = hb((size_t)L * M * kFFN);
  w->NF = hb(M * kD);
  w->RF = f(M);
  w->V = f(M * kAD);
  w->dv = f(M * kAD);
  w->dh = f(M * kD);
  w->dn = f(M * kD);
  w->dact = f(M * kFFN);
  w->dgu = hb(M * kGU);
  w->dh16 = hb(M * kD);
  w->dqkv16 = hb(M * kNQKV);
  w->dout = f(M * kNQ);
  w->dqkv = f(M * kNQKV);
  w->dkv = f((size_t)B * kHQ * 2 * kChunk * kHD);
  w->part = f(nblk * kGU + M);
  w->split = f(train_split_cap(B));
  w->split2 = f(train_split_cap(B));  // the side stream's
  w->vidx = (int*)f((size_t)B * P);
  w->nval = (int*)f(B);
  return off;
}

hipError_t train_enqueue(const TrainArgs& t, hipStream_t st) {
  const int B = t.B, L = t.L, M = B * kChunk, nblk = (M + kRB - 1) / kRB;
  const TrainWs& w = t.ws;
  const bf16_t* W = t.w;
  float* G = t.grads;
  TrOffsets off;
  train_offsets(L, 0, &off);
  hipError_t e;
#define TR_CHECK() do { if ((e = hipGetLastError()) != hipSuccess) return e; } while (0)
  auto gemm_on = [&](hipStream_t gs, float* scratch, int m, int n, int k, const void* A, int lda, bool ak, bool abf,
                     const void* Bp, int ldb, bool bk, bool bbf, float* C, int ldc, const float* cin, const float* bias) {
    TrGemm g;
    g.M = m; g.N = n; g.K = k; g.A = A; g.lda = lda; g.B = Bp; g.ldb = ldb; g.C = C; g.ldc = ldc;
    g.Cin = cin; g.bias = bias; g.alpha = 1.f; g.part = scratch; g.part_cap = t.split_cap;
    return launch_tr_gemm(g, ak, abf, bk, bbf, gs);
  };
  auto gemm = [&](int m, int n, int k, const void* A, int lda, bool ak, bool abf, const void* Bp, int ldb, bool bk,
                  bool bbf, float* C, int ldc, const float* cin, const float* bias) {
    return gemm_on(st, w.split, m, n, k, A, lda, ak, abf, Bp, ldb, bk, bbf, C, ldc, cin, bias);
  };
  // y W^T (+ cin) (+ bias): activations (fp32, or the bf16 the product reads) along k, weights bf16 [out][in]
  auto fwd = [&](const void* x, bool xbf, int ldx, size_t woff, int n, int k, float* y, int ldy, const float* cin,
                 const float* bias) { return gemm(M, n, k, x, ldx, true, xbf, W + woff, k, true, true, y, ldy, cin, bias); };
  // dx = dy W: W [n_out][k_in] read across its rows; dy fp32 or bf16
  auto bwd_x = [&](const void* dy, bool dybf, int n_out, size_t woff, int k_in, int ldw, float* dx) {
    return gemm(M, k_in, n_out, dy, n_out, true, dybf, W + woff, ldw, false, true, dx, k_in, nullptr, nullptr);
  };
  // dW [n_out][k_in] = dy^T x over the M rows (dy's rows ldy wide; dy and x fp32 or bf16)
  auto bwd_w = [&](const void* dy, bool dybf, int ldy, int n_out, const void* x, bool xbf, int k_in, size_t goff) {
    return gemm(n_out, k_in, M, dy, ldy, false, dybf, x, k_in, false, xbf, G + goff, k_in, nullptr, nullptr);
  };
  // The layers' weight gradients only feed the output: they run on the side stream, forked
  // after their operands are written and joined before the main stream overwrites them.
  int nev = 0;
  auto fork = [&]() -> hipError_t {
    if (nev >= t.n_ev) return hipErrorInvalidValue;
    hipEvent_t ev = t.ev[nev++];
    hipError_t r = hipEventRecord(ev, st);
    return r == hipSuccess ? hipStreamWaitEvent(t.side, ev, 0) : r;
  };
  auto side_w = [&](const void* dy, int ldy, int n_out, const void* x, int k_in, size_t goff, hipEvent_t* done) -> hipError_t {
    hipError_t r = fork();
    if (r != hipSuccess) return r;
    r = gemm_on(t.side, w.split2, n_out, k_in, M, dy, ldy, false, true, x, k_in, false, true, G + goff, k_in, nullptr,
                nullptr);
    if (r != hipSuccess) return r;
    if (nev >= t.n_ev) return hipErrorInvalidValue;
    *done = t.ev[nev++];
    return hipEventRecord(*done, t.side);
  };
  auto join = [&](hipEvent_t& ev) -> hipError_t {
    if (!ev) return hipSuccess;
    hipError_t r = hipStreamWaitEvent(st, ev, 0);
    ev = nullptr;
    return r;
  };
  auto colsum = [&](const float* x, int n, float* out) -> hipError_t {
    hipLaunchKernelGGL(tr_colsum_kernel, dim3((n + 255) / 256, nblk), dim3(256), 0, st, x, M, n, w.part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_reduce_kernel, dim3((n + 15) / 16), dim3(256), 0, st, w.part, nblk, n, out);
    return hipGetLastError();
  };
  auto norm_bwd = [&](const float* dy, const float* h, const float* r, size_t goff, const float* resid, float* dh) -> hipError_t {
    hipLaunchKernelGGL(tr_rmsnorm_bwd_kernel, dim3(nblk), dim3(256), 0, st, dy, h, r, W + goff, resid, dh, w.dh16, M, w.part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_reduce_kernel, dim3((kD + 15) / 16), dim3(256), 0, st, w.part, nblk, kD, G + goff);
    return hipGetLastError();
  };
  auto Hl = [&](int l) { return w.H + (size_t)l * M * kD; };
  auto lay = [&](float* base, int l, size_t per_row) { return base + (size_t)l * M * per_row; };
  auto lay16 = [&](bf16_t* base, int l, size_t per_row) { return base + (size_t)l * M * per_row; };

  // ---- forward
  hipLaunchKernelGGL(tr_prep_kernel, dim3(B), dim3(64), 0, st, t.mask, t.P, w.vidx, w.nval);
  TR_CHECK();
  hipLaunchKernelGGL(tr_input_kernel, dim3(M), dim3(256), 0, st, t.actions, t.noise, t.t, t.inv_period, w.xt,
                     w.target, w.z);
  TR_CHECK();
  // the four biases come widened to fp32 (bias32: b_in, b_t1, b_t2, b_out)
  if ((e = fwd(w.xt, false, kAD, off.ain_w, kD, kAD, w.z, 2 * kD, nullptr, t.bias32 + 0)) != hipSuccess) return e;
  if ((e = fwd(w.z, false, 2 * kD, off.tin_w, kD, 2 * kD, w.s, kD, nullptr, t.bias32 + kD)) != hipSuccess) return e;
  hipLaunchKernelGGL(tr_silu_kernel, dim3(ew_grid((size_t)M * kD)), dim3(256), 0, st, w.s, w.sil, (size_t)M * kD);
  TR_CHECK();
  if ((e = fwd(w.sil, true, kD, off.tout_w, kD, kD, Hl(0), kD, nullptr, t.bias32 + 2 * kD)) != hipSuccess) return e;
  for (int l = 0; l < L; ++l) {
    TrOffsets ol;
    train_offsets(L, l, &ol);
    const TrLayerOffsets& lo = ol.layer;
    const bool self = l % 2 == 0;
    const int nq = self ? kNQKV : kNQ;
    float *r1 = w.R1 + (size_t)l * M, *qkv = lay(w.QKV, l, kNQKV), *o = lay(w.O, l, kNQ);
    float *hm = lay(w.HM, l, kD), *r2 = w.R2 + (size_t)l * M, *gu = lay(w.GU, l, kGU);
    bf16_t *n1 = lay16(w.N1, l, kD), *n2 = lay16(w.N2, l, kD), *act = lay16(w.ACT, l, kFFN), *o16 = lay16(w.O16, l, kNQ);
    hipLaunchKernelGGL(tr_rmsnorm_kernel, dim3((M + 3) / 4), dim3(256), 0, st, Hl(l), W + lo.norm1, t.rms_eps, M, n1, r1);
    TR_CHECK();
    if ((e = fwd(n1, true, kD, lo.qkv, nq, kD, qkv, kNQKV, nullptr, nullptr)) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_rope_kernel, dim3(M), dim3(256), 0, st, qkv, kNQKV, self ? kHQ + kHKV : kHQ, w.nval, t.rope, 1.f,
                       nullptr);
    TR_CHECK();
    TrAttn aa;
    aa.qkv = qkv; aa.ldq = kNQKV;
    aa.pk = t.kv + (size_t)l * 2 * B * kHKV * t.P * kHD;
    aa.pv = aa.pk + (size_t)B * kHKV * t.P * kHD;
    aa.vidx = w.vidx; aa.nval = w.nval; aa.P = t.P;
    aa.o = o; aa.o16 = o16; aa.lse = w.LSE + (size_t)l * B * kHQ * kChunk;
    aa.dout = nullptr; aa.dq = nullptr; aa.dkv = nullptr;
    if (self) hipLaunchKernelGGL(tr_attn_fwd_kernel<true>, dim3(kHQ, B), dim3(256), 0, st, aa);
    else hipLaunchKernelGGL(tr_attn_fwd_kernel<false>, dim3(kHQ, B), dim3(256), 0, st, aa);
    TR_CHECK();
    if ((e = fwd(o16, true, kNQ, lo.o, kD, kNQ, hm, kD, Hl(l), nullptr)) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_rmsnorm_kernel, dim3((M + 3) / 4), dim3(256), 0, st, hm, W + lo.norm2, t.rms_eps, M, n2, r2);
    TR_CHECK();
    if ((e = fwd(n2, true, kD, lo.gu, kGU, kD, gu, kGU, nullptr, nullptr)) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_swiglu_kernel, dim3(ew_grid((size_t)M * kFFN / 4)), dim3(256), 0, st, gu, act, (size_t)M * kFFN);
    TR_CHECK();
    if ((e = fwd(act, true, kFFN, lo.down, kD, kFFN, Hl(l + 1), kD, hm, nullptr)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tr_rmsnorm_kernel, dim3((M + 3) / 4), dim3(256), 0, st, Hl(L), W + off.fnorm, t.rms_eps, M, w.NF, w.RF);
  TR_CHECK();
  if ((e = fwd(w.NF, true, kD, off.aout_w, kAD, kD, w.V, kAD, nullptr, t.bias32 + 3 * kD)) != hipSuccess) return e;
  // ---- loss
  const int lblk = (M + 7) / 8;
  hipLaunchKernelGGL(tr_loss_kernel, dim3(lblk), dim3(256), 0, st, w.V, w.target, M, 1.f / ((float)M * kAD), w.dv,
                     w.part);
  TR_CHECK();
  hipLaunchKernelGGL(tr_reduce_kernel, dim3(1), dim3(256), 0, st, w.part, lblk, 1, t.loss);
  TR_CHECK();
  hipLaunchKernelGGL(tr_scale_kernel, dim3(1), dim3(1), 0, st, t.loss, 1.f / ((float)M * kAD));
  TR_CHECK();
  // ---- backward
  if ((e = bwd_w(w.dv, false, kAD, kAD, w.NF, true, kD, off.aout_w)) != hipSuccess) return e;
  if ((e = colsum(w.dv, kAD, G + off.aout_b)) != hipSuccess) return e;
  if ((e = bwd_x(w.dv, false, kAD, off.aout_w, kD, kD, w.dn)) != hipSuccess) return e;
  if ((e = norm_bwd(w.dn, Hl(L), w.RF, off.fnorm, nullptr, w.dh)) != hipSuccess) return e;
  hipEvent_t j_down = nullptr, j_gu = nullptr, j_o = nullptr, j_qkv = nullptr;  // side-stream work in flight
  for (int l = L - 1; l >= 0; --l) {
    TrOffsets ol;
    train_offsets(L, l, &ol);
    const TrLayerOffsets& lo = ol.layer;
    const bool self = l % 2 == 0;
    const int nq = self ? kNQKV : kNQ;
    float *r1 = w.R1 + (size_t)l * M, *qkv = lay(w.QKV, l, kNQKV), *o = lay(w.O, l, kNQ);
    float *hm = lay(w.HM, l, kD), *r2 = w.R2 + (size_t)l * M, *gu = lay(w.GU, l, kGU);
    bf16_t *n1 = lay16(w.N1, l, kD), *n2 = lay16(w.N2, l, kD), *act = lay16(w.ACT, l, kFFN), *o16 = lay16(w.O16, l, kNQ);
    // MLP
    if ((e = bwd_x(w.dh16, true, kD, lo.down, kFFN, kFFN, w.dact)) != hipSuccess) return e;
    if ((e = side_w(w.dh16, kD, kD, act, kFFN, lo.down, &j_down)) != hipSuccess) return e;
    if ((e = join(j_gu)) != hipSuccess) return e;  // the previous layer's gate/up gradient read dgu
    hipLaunchKernelGGL(tr_swiglu_bwd_kernel, dim3(ew_grid((size_t)M * kFFN / 4)), dim3(256), 0, st, w.dact, gu, w.dgu,
                       (size_t)M * kFFN);
    TR_CHECK();
    if ((e = bwd_x(w.dgu, true, kGU, lo.gu, kD, kD, w.dn)) != hipSuccess) return e;
    if ((e = side_w(w.dgu, kGU, kGU, n2, kD, lo.gu, &j_gu)) != hipSuccess) return e;
    if ((e = join(j_down)) != hipSuccess) return e;  // dh16 is about to change
    if ((e = norm_bwd(w.dn, hm, r2, lo.norm2, w.dh, w.dh)) != hipSuccess) return e;  // dh <- d(hm)
    // attention
    if ((e = bwd_x(w.dh16, true, kD, lo.o, kNQ, kNQ, w.dout)) != hipSuccess) return e;
    if ((e = side_w(w.dh16, kD, kD, o16, kNQ, lo.o, &j_o)) != hipSuccess) return e;
    TrAttn aa;
    aa.qkv = qkv; aa.ldq = kNQKV;
    aa.pk = t.kv + (size_t)l * 2 * B * kHKV * t.P * kHD;
    aa.pv = aa.pk + (size_t)B * kHKV * t.P * kHD;
    aa.vidx = w.vidx; aa.nval = w.nval; aa.P = t.P;
    aa.o = o; aa.o16 = nullptr; aa.lse = w.LSE + (size_t)l * B * kHQ * kChunk;
    aa.dout = w.dout; aa.dq = w.dqkv; aa.dkv = w.dkv;
    if (self) hipLaunchKernelGGL(tr_attn_bwd_kernel<true>, dim3(kHQ, B), dim3(256), 0, st, aa);
    else hipLaunchKernelGGL(tr_attn_bwd_kernel<false>, dim3(kHQ, B), dim3(256), 0, st, aa);
    TR_CHECK();
    if ((e = join(j_qkv)) != hipSuccess) return e;  // the previous layer's Q/K/V gradient read dqkv16
    hipLaunchKernelGGL(tr_rope_kernel, dim3(M), dim3(256), 0, st, w.dqkv, kNQKV, kHQ, w.nval, t.rope, -1.f, w.dqkv16);
    TR_CHECK();
    if (self) {
      hipLaunchKernelGGL(tr_kv_grad_kernel, dim3(M), dim3(256), 0, st, w.dkv, w.nval, t.rope, w.dqkv16);
      TR_CHECK();
    }
    if ((e = gemm(M, kD, nq, w.dqkv16, kNQKV, true, true, W + lo.qkv, kD, false, true, w.dn, kD, nullptr, nullptr)) != hipSuccess)
      return e;
    if ((e = side_w(w.dqkv16, kNQKV, nq, n1, kD, lo.qkv, &j_qkv)) != hipSuccess) return e;
    if ((e = join(j_o)) != hipSuccess) return e;  // dh16 is about to change
    if ((e = norm_bwd(w.dn, Hl(l), r1, lo.norm1, w.dh, w.dh)) != hipSuccess) return e;  // dh <- d(h_l)
  }
  // everything on the side stream has finished before the step ends
  if ((e = join(j_gu)) != hipSuccess) return e;
  if ((e = join(j_qkv)) != hipSuccess) return e;
  // time MLP and action_in (dh = d h0)
  if ((e = bwd_w(w.dh16, true, kD, kD, w.sil, true, kD, off.tout_w)) != hipSuccess) return e;
  if ((e = colsum(w.dh, kD, G + off.tout_b)) != hipSuccess) return e;
  if ((e = bwd_x(w.dh16, true, kD, off.tout_w, kD, kD, w.dn)) != hipSuccess) return e;
  hipLaunchKernelGGL(tr_silu_bwd_kernel, dim3(ew_grid((size_t)M * kD)), dim3(256), 0, st, w.dn, w.s, w.dn, (size_t)M * kD);
  TR_CHECK();
  if ((e = bwd_w(w.dn, false, kD, kD, w.z, false, 2 * kD, off.tin_w)) != hipSuccess) return e;
  if ((e = colsum(w.dn, kD, G + off.tin_b)) != hipSuccess) return e;
  // dy = ds W_t1[:, :720]
  if ((e = gemm(M, kD, kD, w.dn, kD, true, false, W + off.tin_w, 2 * kD, false, true, w.dh, kD, nullptr, nullptr)) != hipSuccess)
    return e;
  if ((e = bwd_w(w.dh, false, kD, kD, w.xt, false, kAD, off.ain_w)) != hipSuccess) return e;
  if ((e = colsum(w.dh, kD, G + off.ain_b)) != hipSuccess) return e;
#undef TR_CHECK
  return hipSuccess;
}

}  // namespace smolexp
