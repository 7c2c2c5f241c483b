// HIP kernels of the action-expert denoising loop, written for gfx950 (CDNA4).
//
// GEMMs: C[M,N] = A[M,K] * W[N,K]^T with both operands K-contiguous, on
//   v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulate).  Weights are the
//   checkpoint's bf16 values re-encoded exactly in fp16 with a power-of-two
//   scale per matrix; activations are rounded to fp16 (8x finer than bf16).
//   The A-operand load fuses RMSNorm (row scale from partial sums of squares
//   that the producer of the residual stream wrote) or the prefix overwrite;
//   epilogues fuse bias, SiLU, RoPE, SwiGLU, the residual add and the Euler
//   update.
// Attention: block-masked grouped-query attention on v_mfma_f32_16x16x32_bf16
//   over the bf16 prefix K/V cache and the chunk's own K/V, with an online
//   softmax in fp32 and 64-key blocks staged in LDS.
//
// Sources for what is computed: noeira docs "SmolVLA" (Architecture table and
// paragraphs on the query, the flow-matching objective and the block mask);
// "Paper vs hardware 11: SmolVLA" (What the paper claims: causal
// self-attention over the chunk; What I ran: prefix overwrite).
#include "smolexp_internal.h"

#include <math.h>

namespace smolexp {

typedef half_t f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint4 pack8(const float* v) {
  union { half_t h[8]; uint4 u; } p;
#pragma unroll
  for (int e = 0; e < 8; ++e) p.h[e] = (half_t)v[e];
  return p.u;
}

// ----------------------------------------------------------------------------
// GEMM
// ----------------------------------------------------------------------------
// Two kernels share the A-operand loaders and the epilogues:
//  * gemm_skinny (M <= 64, one query): one 512-thread workgroup per 16 output
//    columns.  Its 8 waves split K; each wave issues every load it needs (its
//    weight fragments and A fragments) at once, so the kernel waits for memory
//    about once, then the waves' partial tiles meet in LDS.
//  * gemm_tiled (M > 64): 128 x 128 output tiles, four waves of 64 x 64,
//    BK = 64 slabs double-buffered in LDS.
// Epilogues run on the finished fp32 tile staged in LDS.
//
// Weight row order inside each 16-row block (set by the host when it loads
// the weights) keeps every pair an epilogue needs in one block:
//  * Q and K heads: block q of a head holds dims q*8..q*8+7, then 32+q*8..
//    32+q*8+7, so column e pairs with e+8 for the rotation of (d, d+32);
//  * gate/up: block j holds gate rows 8j..8j+7, then up rows 8j..8j+7;
//  * V heads and every other matrix keep their natural order.

// Eight consecutive A elements of row `row`, columns k..k+7, converted to the
// fp16 MFMA operand (ok = inside the matrix; otherwise zeros).
template <int AM>
__device__ __forceinline__ uint4 load_a8(const GemmArgs& a, int row, int k, bool ok, float rscale,
                                         bool write_x) {
  if constexpr (AM == A_F16) {
    return ok ? *reinterpret_cast<const uint4*>(static_cast<const half_t*>(a.A) + (size_t)row * a.lda + k)
              : make_uint4(0, 0, 0, 0);
  } else if constexpr (AM == A_NORM) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
      const float* p = static_cast<const float*>(a.A) + (size_t)row * a.lda + k;
      const float4 h0 = *reinterpret_cast<const float4*>(p), h1 = *reinterpret_cast<const float4*>(p + 4);
      const float4 g0 = *reinterpret_cast<const float4*>(a.gain + k), g1 = *reinterpret_cast<const float4*>(a.gain + k + 4);
      v[0] = h0.x * rscale * g0.x; v[1] = h0.y * rscale * g0.y; v[2] = h0.z * rscale * g0.z; v[3] = h0.w * rscale * g0.w;
      v[4] = h1.x * rscale * g1.x; v[5] = h1.y * rscale * g1.y; v[6] = h1.z * rscale * g1.z; v[7] = h1.w * rscale * g1.w;
    }
    return pack8(v);
  } else {  // A_X: Euler state; rows i < ow_rows of each chunk take the flow-path point t*eps + (1-t)*prev
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (ok) {
      const int ci = row % kChunk;
      if (ci < a.ow_rows) {
        const int b = row / kChunk;
        const float* ep = a.noise + (size_t)row * kAD + k;
        const float* pp = a.prev + ((size_t)b * a.ow_rows + ci) * kAD + k;
        const float4 e0 = *reinterpret_cast<const float4*>(ep), e1 = *reinterpret_cast<const float4*>(ep + 4);
        const float4 p0 = *reinterpret_cast<const float4*>(pp), p1 = *reinterpret_cast<const float4*>(pp + 4);
        const float t = a.t, u = 1.0f - a.t;
        v0 = make_float4(t * e0.x + u * p0.x, t * e0.y + u * p0.y, t * e0.z + u * p0.z, t * e0.w + u * p0.w);
        v1 = make_float4(t * e1.x + u * p1.x, t * e1.y + u * p1.y, t * e1.z + u * p1.z, t * e1.w + u * p1.w);
        if (write_x) {  // one workgroup column stores the overwritten rows into the state
          float* xp = a.x + (size_t)row * kAD + k;
          *reinterpret_cast<float4*>(xp) = v0;
          *reinterpret_cast<float4*>(xp + 4) = v1;
        }
      } else {
        const float* p = static_cast<const float*>(a.A) + (size_t)row * a.lda + k;
        v0 = *reinterpret_cast<const float4*>(p);
        v1 = *reinterpret_cast<const float4*>(p + 4);
      }
    }
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    return pack8(v);
  }
}

// RMSNorm row scales 1/sqrt(mean(h^2) + eps) for rows m0..m0+BM-1 from the
// producer's per-N-tile partial sums of squares.  NT/BM threads share a row
// and sum every (NT/BM)-th partial, so the loads are issued side by side.
template <int BM, int NT>
__device__ __forceinline__ void row_scales(const GemmArgs& a, int m0, float* sR) {
  constexpr int TPR = NT / BM;
  static_assert(TPR >= 1 && TPR <= 64 && (TPR & (TPR - 1)) == 0, "threads per row: a power of two within a wave");
  const int r = threadIdx.x / TPR, part = threadIdx.x % TPR, row = m0 + r;
  float s = 0.f;
  if (row < a.M) {
    const float* src = a.ss_in + (size_t)row * kSSStride;
#pragma unroll
    for (int j0 = 0; j0 < kSSStride; j0 += TPR) {
      const int j = j0 + part;
      if (j < a.ss_nt) s += src[j];
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (part == 0) sR[r] = 1.0f / sqrtf(s * a.inv_k + a.eps);
}

// Epilogue on a finished tile sC[BM][LDC] (fp32, weight scale applied) whose
// rows start at m0 and columns at n0 (BN a multiple of 16).  Work unit =
// (row, 16-column block, e < 8) covering columns e and e + 8 of the block;
// the units of one row are consecutive lanes of one wave.  ntile = this
// tile's sum-of-squares slot.
template <int EM, int BM, int BN, int LDC, int NT>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const float* sC, int m0, int n0, int ntile) {
  constexpr int NB = BN / 16, UPR = NB * 8;
  static_assert(UPR <= 64 && 64 % UPR == 0 && (BM * UPR) % NT == 0, "rows inside one wave, uniform trip count");
  const int M = a.M, N = a.N;
  for (int g = threadIdx.x; g < BM * UPR; g += NT) {
    const int r = g / UPR, blk = (g % UPR) / 8, e = g % 8;
    const int row = m0 + r, cb = n0 + blk * 16;
    const bool ok = row < M && cb < N;
    const float v1 = sC[r * LDC + blk * 16 + e], v2 = sC[r * LDC + blk * 16 + 8 + e];
    float ss = 0.f;
    if (ok) {
      if constexpr (EM == E_QKV) {
        const int head = cb / kHD, b = row / kChunk, ci = row % kChunk;
        bf16_t* dst;
        if (head < kHQ) dst = a.q + (((size_t)b * kHQ + head) * kChunk + ci) * kHD;
        else if (head < kHQ + kHKV) dst = a.kc + (((size_t)b * kHKV + head - kHQ) * kChunk + ci) * kHD;
        else dst = a.vc + (((size_t)b * kHKV + head - kHQ - kHKV) * kChunk + ci) * kHD;
        if (head < kHQ + kHKV) {  // rotate the pair (d, d + 32) at position n_valid + i
          const int d = ((cb % kHD) / 16) * 8 + e;
          const float2 cs = a.rope[(size_t)(a.nvalid[b] + ci) * (kHD / 2) + d];
          dst[d] = f2bf(v1 * cs.x - v2 * cs.y);
          dst[d + kHD / 2] = f2bf(v1 * cs.y + v2 * cs.x);
        } else {
          const int d = cb % kHD + e;
          dst[d] = f2bf(v1);
          dst[d + 8] = f2bf(v2);
        }
      } else if constexpr (EM == E_SWIGLU) {
        a.out16[(size_t)row * a.ldo + cb / 2 + e] = (half_t)(silu(v1) * v2);
      } else if constexpr (EM == E_F16_BIAS || EM == E_TIMEIN) {
        const float z1 = v1 + a.bias[cb + e], z2 = v2 + a.bias[cb + 8 + e];
        half_t* o = a.out16 + (size_t)row * a.ldo + cb + e;
        o[0] = (half_t)(EM == E_TIMEIN ? silu(z1) : z1);
        o[8] = (half_t)(EM == E_TIMEIN ? silu(z2) : z2);
      } else if constexpr (EM == E_H_BIAS || EM == E_H_RESID) {
        float* hp = a.h + (size_t)row * kD + cb + e;
        const float h1 = (EM == E_H_BIAS) ? v1 + a.bias[cb + e] : hp[0] + v1;
        const float h2 = (EM == E_H_BIAS) ? v2 + a.bias[cb + 8 + e] : hp[8] + v2;
        hp[0] = h1;
        hp[8] = h2;
        ss = h1 * h1 + h2 * h2;
      } else if constexpr (EM == E_ACTOUT) {
        const size_t xi = (size_t)row * kAD + cb + e;
        const float u1 = v1 + a.bias[cb + e], u2 = v2 + a.bias[cb + 8 + e];
        const float x1 = a.x[xi] + a.dt * u1, x2 = a.x[xi + 8] + a.dt * u2;
        a.x[xi] = x1;
        a.x[xi + 8] = x2;
        if (a.vel_out) { a.vel_out[xi] = u1; a.vel_out[xi + 8] = u2; }
        if (a.st_out) { a.st_out[xi] = x1; a.st_out[xi + 8] = x2; }
        if (a.final_out) { a.final_out[xi] = x1; a.final_out[xi + 8] = x2; }
      }
    }
    if constexpr (EM == E_H_BIAS || EM == E_H_RESID) {
#pragma unroll
      for (int off = UPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      if (g % UPR == 0 && row < M) a.ss_out[(size_t)row * kSSStride + ntile] = ss;
    }
  }
}

// M <= 64.  One workgroup per 16 output columns; wave w takes k-steps
// w*KPW .. w*KPW+KPW-1 (32 wide each).
template <int AM, int EM, int KPW>
__global__ __launch_bounds__(512) void gemm_skinny(const GemmArgs a) {
  constexpr int NW = 8, LDC = 16;
  __shared__ float sRed[NW * 64 * 16];
  __shared__ float sC[64 * LDC];
  __shared__ float sR[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int M = a.M, N = a.N, K = a.K;
  const int nks = (K + 31) / 32;
  const int n = n0 + (lane & 15), kl = (lane >> 4) * 8;

  uint4 wf[KPW];
  uint4 af[KPW][4];
  float4 ra[AM == A_NORM ? KPW : 1][4][2];
  float4 gv[AM == A_NORM ? KPW : 1][2];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = w * KPW + i, k = ks * 32 + kl;
    const bool kok = ks < nks && k < K;
    wf[i] = (kok && n < N) ? *reinterpret_cast<const uint4*>(a.W + (size_t)n * a.ldw + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int row = fm * 16 + (lane & 15);
      const bool ok = kok && row < M;
      if constexpr (AM == A_NORM) {
        const float* p = static_cast<const float*>(a.A) + (size_t)row * a.lda + k;
        ra[i][fm][0] = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
        ra[i][fm][1] = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        af[i][fm] = load_a8<AM>(a, row, k, ok, 1.f, blockIdx.x == 0);
      }
    }
    if constexpr (AM == A_NORM) {
      gv[i][0] = kok ? *reinterpret_cast<const float4*>(a.gain + k) : make_float4(0.f, 0.f, 0.f, 0.f);
      gv[i][1] = kok ? *reinterpret_cast<const float4*>(a.gain + k + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if constexpr (AM == A_NORM) {
    row_scales<64, 512>(a, 0, sR);
    __syncthreads();
  }
  f32x4 acc[4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) acc[fm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const f16x8 bw = __builtin_bit_cast(f16x8, wf[i]);
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      uint4 frag;
      if constexpr (AM == A_NORM) {
        const float sc = sR[fm * 16 + (lane & 15)];
        const float v[8] = {ra[i][fm][0].x * sc * gv[i][0].x, ra[i][fm][0].y * sc * gv[i][0].y,
                            ra[i][fm][0].z * sc * gv[i][0].z, ra[i][fm][0].w * sc * gv[i][0].w,
                            ra[i][fm][1].x * sc * gv[i][1].x, ra[i][fm][1].y * sc * gv[i][1].y,
                            ra[i][fm][1].z * sc * gv[i][1].z, ra[i][fm][1].w * sc * gv[i][1].w};
        frag = pack8(v);
      } else {
        frag = af[i][fm];
      }
      acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, frag), bw, acc[fm], 0, 0, 0);
    }
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) sRed[(w * 64 + fm * 16 + (lane >> 4) * 4 + r) * 16 + (lane & 15)] = acc[fm][r];
  __syncthreads();
  const float ws = a.w_scale;
  for (int i = tid; i < 64 * 16; i += 512) {
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) s += sRed[w2 * 64 * 16 + i];
    sC[(i / 16) * LDC + (i % 16)] = s * ws;
  }
  __syncthreads();
  epilogue_tile<EM, 64, 16, LDC, 512>(a, sC, 0, n0, blockIdx.x);
}

// FM = 16-row MFMA tiles per wave along M: BM = 32 * FM rows (two waves along M).
template <int AM, int EM, int FM>
__global__ __launch_bounds__(256, 2) void gemm_tiled(const GemmArgs a) {
  constexpr int BM = 32 * FM, BN = 128, BK = 64, LDK = BK + 8, LDC = BN + 4, CPR = BK / 8;
  constexpr int GA = BM * CPR / 256, GW = BN * CPR / 256;
  constexpr int STAGE = (BM + BN) * LDK;  // halves
  constexpr int SMEM = 2 * STAGE * 2 > BM * LDC * 4 ? 2 * STAGE * 2 : BM * LDC * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ float sR[BM];
  __shared__ float sG[AM == A_NORM ? kD : 1];
  half_t* stage0 = reinterpret_cast<half_t*>(smem);
  float* sC = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int M = a.M, N = a.N, K = a.K;
  // XCD-aware tile order: workgroups are dispatched to the 8 XCDs round-robin,
  // so workgroup id goes to XCD id % 8.  XCD x takes the contiguous range
  // [x * per, (x + 1) * per) of the M-major tile order, i.e. a few row panels of
  // A with all of their N tiles, and keeps those A panels in its own L2.
  const int nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN, T = nM * nN;
  const int per = (T + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (tile >= T) return;  // uniform per workgroup, before any barrier
  const int mt = tile / nN, nt = tile % nN;
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk = (K + BK - 1) / BK;

  if constexpr (AM == A_NORM) {
    row_scales<BM, 256>(a, m0, sR);
    for (int k = tid; k < K; k += 256) sG[k] = a.gain[k];
    __syncthreads();
  }
  uint4 ra[GA], rw[GW];
  float4 rf[AM == A_NORM ? 2 * GA : 1];  // A_NORM: raw fp32 rows, converted when stored to LDS
  auto load = [&](int kt) {
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < GA; ++i) {
      const int g = tid + 256 * i, r = g / CPR, c = (g % CPR) * 8, row = m0 + r, k = kb + c;
      const bool ok = row < M && k < K;
      if constexpr (AM == A_NORM) {
        const float* p = static_cast<const float*>(a.A) + (size_t)row * a.lda + k;
        rf[2 * i] = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
        rf[2 * i + 1] = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        ra[i] = load_a8<AM>(a, row, k, ok, 1.f, nt == 0);
      }
    }
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = tid + 256 * i, r = g / CPR, c = (g % CPR) * 8, n = n0 + r, k = kb + c;
      rw[i] = (n < N && k < K) ? *reinterpret_cast<const uint4*>(a.W + (size_t)n * a.ldw + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf, int kt) {
    half_t* sA = stage0 + buf * STAGE;
    half_t* sW = sA + BM * LDK;
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < GA; ++i) {
      const int g = tid + 256 * i, r = g / CPR, c = (g % CPR) * 8;
      uint4 v;
      if constexpr (AM == A_NORM) {
        const float sc = sR[r];
        const int k = kb + c;
        const bool kin = k < K;
        float f[8] = {rf[2 * i].x, rf[2 * i].y, rf[2 * i].z, rf[2 * i].w,
                      rf[2 * i + 1].x, rf[2 * i + 1].y, rf[2 * i + 1].z, rf[2 * i + 1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = kin ? f[e] * sc * sG[k + e] : 0.f;
        v = pack8(f);
      } else {
        v = ra[i];
      }
      *reinterpret_cast<uint4*>(sA + r * LDK + c) = v;
    }
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = tid + 256 * i;
      *reinterpret_cast<uint4*>(sW + (g / CPR) * LDK + (g % CPR) * 8) = rw[i];
    }
  };

  f32x4 acc[FM][4];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const half_t* sA = stage0 + (kt & 1) * STAGE;
    const half_t* sW = sA + BM * LDK;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      f16x8 af[FM], bw[4];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const f16x8*>(sA + (wm * FM * 16 + fm * 16 + (lane & 15)) * LDK + s * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        bw[fn] = *reinterpret_cast<const f16x8*>(sW + (wn * 64 + fn * 16 + (lane & 15)) * LDK + s * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
    }
    if (kt + 1 < nk) store((kt + 1) & 1, kt + 1);
    __syncthreads();
  }

  const float ws = a.w_scale;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sC[(wm * FM * 16 + fm * 16 + (lane >> 4) * 4 + r) * LDC + wn * 64 + fn * 16 + (lane & 15)] = acc[fm][fn][r] * ws;
  __syncthreads();
  epilogue_tile<EM, BM, BN, LDC, 256>(a, sC, m0, n0, nt);
}

GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p;
  const int nks = (K + 31) / 32;
  p.bm = 64;
  if (M <= 64) {
    p.kind = 0;
    p.ntiles_n = (N + 15) / 16;
    const int need = (nks + 7) / 8;
    p.kpw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 6 ? 6 : need <= 8 ? 8 : 0;
  } else {
    p.kind = 1;
    p.ntiles_n = (N + 127) / 128;
    p.kpw = 0;
    p.bm = N <= 1024 ? 64 : 128;  // measured: 64-row tiles fill the chip better for N = 720/960
  }
  return p;
}

template <int AM, int EM>
static hipError_t launch_gemm_t(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  if (p.kind == 0) {
    const dim3 grid(p.ntiles_n), block(512);
    switch (p.kpw) {
      case 1: hipLaunchKernelGGL((gemm_skinny<AM, EM, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((gemm_skinny<AM, EM, 2>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((gemm_skinny<AM, EM, 3>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((gemm_skinny<AM, EM, 4>), grid, block, 0, s, a); break;
      case 6:
      case 8:
        // only the fp16-operand GEMMs have K > 1024 (down: K = 2048); the fp32-input
        // variants would not fit their fragments in registers
        if constexpr (AM == A_F16) {
          if (p.kpw == 6) hipLaunchKernelGGL((gemm_skinny<AM, EM, 6>), grid, block, 0, s, a);
          else hipLaunchKernelGGL((gemm_skinny<AM, EM, 8>), grid, block, 0, s, a);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;  // K beyond 8 waves x 8 k-steps x 32
    }
  } else {
    const int T = ((a.M + p.bm - 1) / p.bm) * p.ntiles_n;
    const dim3 grid(8 * ((T + 7) / 8));
    if (p.bm == 128) hipLaunchKernelGGL((gemm_tiled<AM, EM, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_tiled<AM, EM, 2>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& p, AMode am, EMode em, const GemmArgs& a, hipStream_t s) {
#define SMOLEXP_GEMM_CASE(AMV, EMV) \
  if (am == AMV && em == EMV) return launch_gemm_t<AMV, EMV>(p, a, s);
  SMOLEXP_GEMM_CASE(A_X, E_F16_BIAS)
  SMOLEXP_GEMM_CASE(A_F16, E_TIMEIN)
  SMOLEXP_GEMM_CASE(A_F16, E_H_BIAS)
  SMOLEXP_GEMM_CASE(A_NORM, E_QKV)
  SMOLEXP_GEMM_CASE(A_F16, E_H_RESID)
  SMOLEXP_GEMM_CASE(A_NORM, E_SWIGLU)
  SMOLEXP_GEMM_CASE(A_NORM, E_ACTOUT)
#undef SMOLEXP_GEMM_CASE
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Block-masked grouped-query attention
// ----------------------------------------------------------------------------
// One workgroup per (query tile of 64 rows, KV head g, query b).  The 150
// query rows of KV head g are its 3 query heads x 50 chunk rows.  Keys are the
// prefix tokens 0..P-1 (valid where the mask says so) followed, in self layers,
// by the 50 chunk keys, of which row i sees j <= i.  Scores are computed
// transposed (S^T = K Q^T) so that each lane owns one query row; the output is
// accumulated transposed as well (O^T += V^T P^T).
constexpr int kKB = 64;        // keys per block
constexpr int kALD = kHD + 8;  // LDS row stride of K (elements)

// One 64-key block of the online softmax for the lane's query row (row qi of
// the chunk).  sKb: the block's K rows [64][kALD]; sVb: its V^T columns
// (row stride vld); kind: its key kinds; key0 = index of its first key minus P
// (chunk key j is visible to row qi when j - P <= qi).
__device__ __forceinline__ void attn_block(const bf16_t* sKb, const bf16_t* sVb, int vld, const uint8_t* kind,
                                           int key0, int qi, const bf16x8* qf, f32x4* o, float& m_run,
                                           float& l_run, int lane) {
  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
  // S^T[key][row] for the 64 keys of the block (4 tiles of 16 keys)
  f32x4 sc[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    sc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = *reinterpret_cast<const uint4*>(sKb + (sub * 16 + (lane & 15)) * kALD + kk * 32 + (lane >> 4) * 8);
      sc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), qf[kk], sc[sub], 0, 0, 0);
    }
  }
  // masks without branches: four key kinds per 32-bit LDS read, bitwise logic
  float mb = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const int jl0 = sub * 16 + (lane >> 4) * 4;
    const unsigned k4 = *reinterpret_cast<const unsigned*>(kind + jl0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned kd = (k4 >> (8 * r)) & 0xffu;
      const bool ok = (kd == 1u) | ((kd == 2u) & ((key0 + jl0 + r) <= qi));
      const float val = ok ? sc[sub][r] * sl2 : -INFINITY;
      sc[sub][r] = val;
      mb = fmaxf(mb, val);
    }
  }
  mb = fmaxf(mb, __shfl_xor(mb, 16));
  mb = fmaxf(mb, __shfl_xor(mb, 32));
  const float m_new = fmaxf(m_run, mb);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  // v_exp_f32 directly: arguments are <= 0 and results that would be
  // denormal may flush to zero, which a softmax weight can afford
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  float ls = 0.f;
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(sc[sub][r] - m_use);
      sc[sub][r] = p;
      ls += p;
    }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  l_run = l_run * alpha + ls;
  m_run = m_new;
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] *= alpha;
  // O^T[d][row] += V^T[d][key] P^T[key][row], 32 keys per MFMA.  The k-slot
  // order (keys 4q..4q+3 then 16+4q..16+4q+3 for lane group q) is the same for
  // both operands.
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    bf16x8 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = (__bf16)sc[2 * h2][r];
      pb[4 + r] = (__bf16)sc[2 * h2 + 1][r];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bf16_t* vp = sVb + (m * 16 + (lane & 15)) * vld + h2 * 32 + (lane >> 4) * 4;
      const uint2 lo = *reinterpret_cast<const uint2*>(vp);
      const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
      const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), pb, o[m], 0, 0, 0);
    }
  }
}

// Stage keys r0 .. r0 + RK - 1 of one (query, KV head) into LDS: K rows,
// V transposed, key kinds.  Branch-free: every address is clamped into its
// buffer and the loaded vector is zeroed afterwards for masked or missing
// keys, so all loads are in flight together.
template <bool SELF, int RK>
__device__ __forceinline__ void attn_stage(const AttnArgs& a, int b, int g, int r0, bf16_t* sK, bf16_t* sVt,
                                           uint8_t* sKind, int nthreads) {
  constexpr int VLD = RK + 8;
  constexpr int NV = RK * 8 / 256;  // 16-byte vectors per thread (256 threads)
  const int tid = threadIdx.x, P = a.P;
  const bf16_t* pk = a.pk + ((size_t)b * kHKV + g) * (size_t)P * kHD;
  const bf16_t* pv = a.pv + ((size_t)b * kHKV + g) * (size_t)P * kHD;
  const bf16_t* ck = SELF ? a.kc + ((size_t)b * kHKV + g) * kChunk * kHD : pk;
  const bf16_t* cv = SELF ? a.vc + ((size_t)b * kHKV + g) * kChunk * kHD : pv;
  const uint8_t* mk = a.mask + (size_t)b * P;
  (void)nthreads;
  for (int i = tid; i < RK; i += 256) {
    const int j = r0 + i;
    sKind[i] = j < P ? (mk[j] ? 1 : 0) : ((SELF && j - P < kChunk) ? 2 : 0);
  }
  uint4 kv[NV], vv[NV];
  bool kok[NV], vok[NV];
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    const int v = tid + 256 * it;
    {  // K rows: 8 lanes per key
      const int j = r0 + (v >> 3), c = (v & 7) * 8;
      const bool pre = j < P, chunk = SELF && !pre && j - P < kChunk;
      const bf16_t* src = pre ? pk + (size_t)j * kHD + c : (chunk ? ck + (size_t)(j - P) * kHD + c : pk + c);
      kv[it] = *reinterpret_cast<const uint4*>(src);
      kok[it] = pre ? mk[j] != 0 : chunk;
    }
    {  // V rows for the transposed store: consecutive lanes take consecutive keys
      const int j = r0 + (v % RK), c = (v / RK) * 8;
      const bool pre = j < P, chunk = SELF && !pre && j - P < kChunk;
      const bf16_t* src = pre ? pv + (size_t)j * kHD + c : (chunk ? cv + (size_t)(j - P) * kHD + c : pv + c);
      vv[it] = *reinterpret_cast<const uint4*>(src);
      vok[it] = pre ? mk[j] != 0 : chunk;
    }
  }
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    if (!kok[it]) kv[it] = make_uint4(0, 0, 0, 0);
    if (!vok[it]) vv[it] = make_uint4(0, 0, 0, 0);
    const int v = tid + 256 * it;
    *reinterpret_cast<uint4*>(sK + (v >> 3) * kALD + (v & 7) * 8) = kv[it];
    const int jl = v % RK, c = (v / RK) * 8;
    const bf16_t* e = reinterpret_cast<const bf16_t*>(&vv[it]);
#pragma unroll
    for (int t = 0; t < 8; ++t) sVt[(c + t) * VLD + jl] = e[t];
  }
}

// NBLK key blocks are staged per round: all of their loads are issued before
// the first is stored, so a round costs one memory round trip.  Small batches
// stage five blocks (320 keys: a whole prefix plus the chunk), large batches
// one block per round and more workgroups per CU.
template <bool SELF, int NBLK>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int RK = NBLK * kKB;     // keys per round
  constexpr int VLD = RK + 8;        // LDS row stride of V^T (elements)
  __shared__ __attribute__((aligned(16))) bf16_t sK[RK * kALD];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kHD * VLD];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[RK];  // 0 = no key, 1 = valid prefix key, 2 = chunk key

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y, b = blockIdx.z;
  const int P = a.P;
  const int rq = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const bool rvalid = rq < 3 * kChunk;
  const int hq = 3 * g + (rvalid ? rq / kChunk : 0);
  const int qi = rvalid ? rq % kChunk : 0;

  bf16x8 qf[2];
  {
    const bf16_t* qp = a.q + (((size_t)b * kHQ + hq) * kChunk + qi) * kHD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = rvalid ? *reinterpret_cast<const uint4*>(qp + kk * 32) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int NK = P + (SELF ? kChunk : 0);
  for (int r0 = 0; r0 < NK; r0 += RK) {
    __syncthreads();  // the previous round's LDS reads are done
    attn_stage<SELF, RK>(a, b, g, r0, sK, sVt, sKind, 256);
    __syncthreads();

    const int nb = min(NBLK, (NK - r0 + kKB - 1) / kKB);
    for (int blk = 0; blk < nb; ++blk)
      attn_block(sK + blk * kKB * kALD, sVt + blk * kKB, VLD, sKind + blk * kKB, r0 + blk * kKB - P, qi, qf, o,
                 m_run, l_run, lane);
  }

  if (rvalid) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    half_t* op = a.out + ((size_t)b * kChunk + qi) * kNQ + hq * kHD + (lane >> 4) * 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int r = 0; r < 4; ++r) pk4.h[r] = (half_t)(o[m][r] * inv);
      *reinterpret_cast<uint2*>(op + m * 16) = pk4.u;
    }
  }
}

// Small batches: the four waves of a workgroup share 16 query rows and split
// the key blocks among themselves (wave w takes blocks w, w + 4, ...), then
// merge their softmax states (running max, running sum, unnormalised output)
// through LDS.  Five times as many workgroups as attn_kernel at batch 1.
template <bool SELF>
__global__ __launch_bounds__(256) void attn_ksplit_kernel(const AttnArgs a) {
  constexpr int NBLK = 5, RK = NBLK * kKB, VLD = RK + 8, OLD = kHD + 4;
  __shared__ __attribute__((aligned(16))) bf16_t sK[RK * kALD];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kHD * VLD];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[RK];
  __shared__ float sM[4][16], sL[4][16];
  float* sO = reinterpret_cast<float*>(sK);  // [4 waves][16 rows][OLD], used after the last round
  static_assert(4 * 16 * OLD * 4 <= (int)sizeof(sK), "merge buffer fits in the K staging area");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y, b = blockIdx.z;
  const int P = a.P;
  const int rq = blockIdx.x * 16 + (lane & 15);
  const bool rvalid = rq < 3 * kChunk;
  const int hq = 3 * g + (rvalid ? rq / kChunk : 0);
  const int qi = rvalid ? rq % kChunk : 0;

  bf16x8 qf[2];
  {
    const bf16_t* qp = a.q + (((size_t)b * kHQ + hq) * kChunk + qi) * kHD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = rvalid ? *reinterpret_cast<const uint4*>(qp + kk * 32) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int NK = P + (SELF ? kChunk : 0);
  for (int r0 = 0; r0 < NK; r0 += RK) {
    __syncthreads();
    attn_stage<SELF, RK>(a, b, g, r0, sK, sVt, sKind, 256);
    __syncthreads();
    const int nb = min(NBLK, (NK - r0 + kKB - 1) / kKB);
    for (int blk = wave; blk < nb; blk += 4)
      attn_block(sK + blk * kKB * kALD, sVt + blk * kKB, VLD, sKind + blk * kKB, r0 + blk * kKB - P, qi, qf, o,
                 m_run, l_run, lane);
  }

  // merge the four waves' states
  __syncthreads();
  if (lane < 16) {
    sM[wave][lane] = m_run;
    sL[wave][lane] = l_run;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(wave * 16 + (lane & 15)) * OLD + m * 16 + (lane >> 4) * 4 + r] = o[m][r];
  __syncthreads();
  {
    const int row = tid >> 4, d0 = (tid & 15) * 4;
    const int rq2 = blockIdx.x * 16 + row;
    if (rq2 < 3 * kChunk) {
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sM[w][row]);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = __builtin_amdgcn_exp2f(sM[w][row] - mu);
        l += sL[w][row] * sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += sO[(w * 16 + row) * OLD + d0 + e] * sc;
      }
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int hq2 = 3 * g + rq2 / kChunk, qi2 = rq2 % kChunk;
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk4.h[e] = (half_t)(acc[e] * inv);
      *reinterpret_cast<uint2*>(a.out + ((size_t)b * kChunk + qi2) * kNQ + hq2 * kHD + d0) = pk4.u;
    }
  }
}

hipError_t launch_attention(bool self_layer, const AttnArgs& a, hipStream_t s) {
  const dim3 block(256);
  if (a.B <= 8) {
    const dim3 grid((3 * kChunk + 15) / 16, kHKV, a.B);
    if (self_layer) hipLaunchKernelGGL(attn_ksplit_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_ksplit_kernel<false>, grid, block, 0, s, a);
  } else {
    const dim3 grid(3, kHKV, a.B);
    if (self_layer) hipLaunchKernelGGL((attn_kernel<true, 1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<false, 1>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Per-call prologue: the time vectors W_t1[:, 720:] e(t_k) + b_t1 for every
// step, the number of valid prefix tokens per query, and x <- the caller's x.
// ----------------------------------------------------------------------------
constexpr int kTimeRowsPerBlock = 16;
constexpr int kTimeBlocks = kD / kTimeRowsPerBlock;  // 45

__global__ __launch_bounds__(256) void prologue_kernel(const PrologueArgs a) {
  __shared__ float se[kD];
  const int tid = threadIdx.x;
  const int nMaskBlocks = (a.B + 3) / 4;
  if (blockIdx.x < kTimeBlocks) {
    // Sinusoidal time embedding: sin(2 pi t / p_i) for i < 360, cos(...) after,
    // periods geometric from p_min to p_max (1/p_i precomputed in fp64).  The
    // angle is reduced to [0, 2 pi) in fp64, then sin/cos run in fp32.
    // Row j of W_t1[:, 720:] is read once, 8 halves per lane, for every step.
    const int j = blockIdx.x * kTimeRowsPerBlock + (tid >> 4), part = tid & 15;
    const half_t* wr = a.w_t1 + (size_t)j * (2 * kD) + kD;
    constexpr int CH = kD / 8;                  // 90 chunks of 8
    constexpr int PER = (CH + 15) / 16;         // 6 chunks per lane
    uint4 wv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = part + 16 * u;
      wv[u] = c < CH ? *reinterpret_cast<const uint4*>(wr + c * 8) : make_uint4(0, 0, 0, 0);
    }
    for (int k = 0; k < a.n_t; ++k) {
      __syncthreads();
      for (int i = tid; i < kD; i += 256) {
        const int halfd = kD / 2, ii = i % halfd;
        const double turns = (double)a.t[k] * a.inv_period[ii];
        const float ang = (float)(6.283185307179586 * (turns - floor(turns)));
        float sn, cs;
        sincosf(ang, &sn, &cs);
        se[i] = i < halfd ? sn : cs;
      }
      __syncthreads();
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = part + 16 * u;
        if (c < CH) {
          const half_t* w8 = reinterpret_cast<const half_t*>(&wv[u]);
#pragma unroll
          for (int e = 0; e < 8; ++e) s += (float)w8[e] * se[c * 8 + e];
        }
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      if (part == 0) a.cvec[(size_t)k * kD + j] = s * a.s_t1 + a.b_t1[j];
    }
  } else if ((int)blockIdx.x < kTimeBlocks + nMaskBlocks) {
    const int b = (blockIdx.x - kTimeBlocks) * 4 + (tid >> 6), lane = tid & 63;
    if (b < a.B) {
      int c = 0;
      for (int j = lane; j < a.P; j += 64) c += a.mask[(size_t)b * a.P + j] != 0;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
      if (lane == 0) a.nvalid[b] = c;
    }
  } else {
    const int first = kTimeBlocks + nMaskBlocks;
    const int n = a.B * kChunk * kAD;
    for (int i = (blockIdx.x - first) * 256 + tid; i < n; i += (gridDim.x - first) * 256) a.x[i] = a.x_in[i];
  }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  const int nMaskBlocks = (a.B + 3) / 4;
  const int nCopy = (a.B * kChunk * kAD + 255) / 256;
  const int copyBlocks = nCopy < 64 ? nCopy : 64;
  hipLaunchKernelGGL(prologue_kernel, dim3(kTimeBlocks + nMaskBlocks + copyBlocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Inverse periods of the time embedding: 1 / (p_min (p_max/p_min)^(i/359)), fp64.
__global__ void inv_period_kernel(double* tab, float p_min, float p_max) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= kD / 2) return;
  const double frac = (double)i / (double)(kD / 2 - 1);
  tab[i] = 1.0 / ((double)p_min * pow((double)p_max / (double)p_min, frac));
}

hipError_t launch_inv_period_table(double* tab, float p_min, float p_max, hipStream_t s) {
  hipLaunchKernelGGL(inv_period_kernel, dim3((kD / 2 + 255) / 256), dim3(256), 0, s, tab, p_min, p_max);
  return hipGetLastError();
}

// RoPE table: (cos, sin) of pos * theta^(-2d/64) for d < 32, fp64 then fp32.
__global__ void rope_table_kernel(float2* tab, int n_pos, float theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pos * (kHD / 2)) return;
  const int pos = i / (kHD / 2), d = i % (kHD / 2);
  const double ang = (double)pos * pow((double)theta, -2.0 * d / kHD);
  tab[i] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2* tab, int n_pos, float theta, hipStream_t s) {
  const int n = n_pos * (kHD / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tab, n_pos, theta);
  return hipGetLastError();
}

}  // namespace smolexp
