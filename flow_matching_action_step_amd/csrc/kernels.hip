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

// Tile: WM x WN x WK waves (4 in total); each wave owns FM x 4 MFMA 16x16
// tiles (16*FM rows x 64 columns) and KS/WK of the KS 32-wide k-steps of a
// BK = 32*KS slab.  With WK > 1 the waves split K and reduce through LDS.
template <int WM_, int WN_, int WK_, int FM_, int KS_>
struct TileT {
  static constexpr int WM = WM_, WN = WN_, WK = WK_, FM = FM_, FN = 4, KS = KS_;
  static constexpr int BM = WM * FM * 16, BN = WN * FN * 16, BK = KS * 32, LDK = BK + 8;
  static constexpr int CPR = BK / 8;              // 8-element chunks per slab row
  static constexpr int GA = BM * BK / 8 / 256;    // A chunks per thread
  static constexpr int GW = BN * BK / 8 / 256;    // W chunks per thread
  static constexpr int TILE_BYTES = (BM + BN) * LDK * 2;
  static constexpr int RED_BYTES = (WK - 1) * WM * WN * FM * FN * 4 * 64 * 4;
  static constexpr int SMEM = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
  static_assert(WM * WN * WK == 4, "four waves");
  static_assert(KS % WK == 0, "k-steps split evenly");
  static_assert(GA * 256 * 8 == BM * BK && GW * 256 * 8 == BN * BK, "whole chunks per thread");
};
using SkinnyTile = TileT<1, 1, 4, 4, 4>;  // 64 x 64, BK 128, K split over the 4 waves
using MedTile = TileT<2, 2, 1, 2, 2>;     // 64 x 128, BK 64

template <class T, int AM, int EM>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[T::SMEM];
  __shared__ float sR[T::BM];
  __shared__ float sSS[T::WN][T::BM];
  half_t* sA = reinterpret_cast<half_t*>(smem);
  half_t* sW = sA + T::BM * T::LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wk = wave % T::WK;
  const int wn = (wave / T::WK) % T::WN;
  const int wm = wave / (T::WK * T::WN);
  const int m0 = blockIdx.x * T::BM, n0 = blockIdx.y * T::BN;
  const int M = a.M, N = a.N, K = a.K;

  if constexpr (AM == A_NORM) {
    // RMSNorm row scale 1/sqrt(mean(h^2) + eps) from the producer's partial sums.
    for (int r = tid; r < T::BM; r += 256) {
      const int row = m0 + r;
      float s = 0.f;
      if (row < M)
        for (int j = 0; j < a.ss_nt; ++j) s += a.ss_in[(size_t)row * kSSStride + j];
      sR[r] = 1.0f / sqrtf(s * a.inv_k + a.eps);
    }
    __syncthreads();
  }

  uint4 ra[T::GA];
  float4 rf[2 * T::GA];
  float4 rg[2 * T::GA];
  uint4 rw[T::GW];

  auto load = [&](int kt) {
    const int kb = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::GA; ++i) {
      const int g = tid + 256 * i, r = g / T::CPR, c = (g % T::CPR) * 8;
      const int row = m0 + r, k = kb + c;
      const bool ok = row < M && k < K;
      if constexpr (AM == A_F16) {
        ra[i] = ok ? *reinterpret_cast<const uint4*>(static_cast<const half_t*>(a.A) + (size_t)row * a.lda + k)
                   : make_uint4(0, 0, 0, 0);
      } else if constexpr (AM == A_NORM) {
        const float* p = static_cast<const float*>(a.A) + (size_t)row * a.lda + k;
        rf[2 * i] = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
        rf[2 * i + 1] = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        rg[2 * i] = ok ? *reinterpret_cast<const float4*>(a.gain + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        rg[2 * i + 1] = ok ? *reinterpret_cast<const float4*>(a.gain + k + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {  // A_X: Euler state, rows i < ow_rows of each chunk replaced by the flow-path point
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
            if (blockIdx.y == 0) {  // the state itself takes the overwritten rows
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
        rf[2 * i] = v0;
        rf[2 * i + 1] = v1;
      }
    }
#pragma unroll
    for (int i = 0; i < T::GW; ++i) {
      const int g = tid + 256 * i, r = g / T::CPR, c = (g % T::CPR) * 8;
      const int n = n0 + r, k = kb + c;
      rw[i] = (n < N && k < K) ? *reinterpret_cast<const uint4*>(a.W + (size_t)n * a.ldw + k)
                               : make_uint4(0, 0, 0, 0);
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < T::GA; ++i) {
      const int g = tid + 256 * i, r = g / T::CPR, c = (g % T::CPR) * 8;
      uint4* dst = reinterpret_cast<uint4*>(sA + r * T::LDK + c);
      if constexpr (AM == A_F16) {
        *dst = ra[i];
      } else {
        float v[8] = {rf[2 * i].x, rf[2 * i].y, rf[2 * i].z, rf[2 * i].w,
                      rf[2 * i + 1].x, rf[2 * i + 1].y, rf[2 * i + 1].z, rf[2 * i + 1].w};
        if constexpr (AM == A_NORM) {
          const float sc = sR[r];
          const float gv[8] = {rg[2 * i].x, rg[2 * i].y, rg[2 * i].z, rg[2 * i].w,
                               rg[2 * i + 1].x, rg[2 * i + 1].y, rg[2 * i + 1].z, rg[2 * i + 1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * sc * gv[e];
        }
        *dst = pack8(v);
      }
    }
#pragma unroll
    for (int i = 0; i < T::GW; ++i) {
      const int g = tid + 256 * i, r = g / T::CPR, c = (g % T::CPR) * 8;
      *reinterpret_cast<uint4*>(sW + r * T::LDK + c) = rw[i];
    }
  };

  f32x4 acc[T::FM][T::FN];
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + T::BK - 1) / T::BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    store();
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < T::KS / T::WK; ++kk) {
      const int ks = kk * T::WK + wk;
      f16x8 af[T::FM], bw[T::FN];
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
        af[fm] = *reinterpret_cast<const f16x8*>(
            sA + (wm * T::FM * 16 + fm * 16 + (lane & 15)) * T::LDK + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn)
        bw[fn] = *reinterpret_cast<const f16x8*>(
            sW + (wn * 64 + fn * 16 + (lane & 15)) * T::LDK + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
    }
    __syncthreads();
  }

  if constexpr (T::WK > 1) {
    // Waves that split K hand their partial tiles to wave wk == 0 through LDS.
    float* red = reinterpret_cast<float*>(smem);
    const int slot = wm * T::WN + wn;
    constexpr int PER = T::FM * T::FN * 4 * 64;
    if (wk > 0) {
      float* dst = red + ((wk - 1) * T::WM * T::WN + slot) * PER;
#pragma unroll
      for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[((fm * T::FN + fn) * 4 + r) * 64 + lane] = acc[fm][fn][r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < T::WK; ++w) {
        const float* src = red + ((w - 1) * T::WM * T::WN + slot) * PER;
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[fm][fn][r] += src[((fm * T::FN + fn) * 4 + r) * 64 + lane];
      }
    }
  }

  // ---------------- epilogue: lane holds C[4*(lane>>4) + r][lane & 15] of each 16x16 tile
  const float ws = a.w_scale;
  const int cbase = n0 + wn * 64;  // first column of this wave (64 wide)
  if (wk == 0) {
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * T::FM * 16 + fm * 16 + (lane >> 4) * 4 + r;
        const int row = m0 + rl;
        const bool rok = row < M;
        if constexpr (EM == E_H_BIAS || EM == E_H_RESID) {
          float ss = 0.f;
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn) {
            const int col = cbase + fn * 16 + (lane & 15);
            if (rok && col < N) {
              float* hp = a.h + (size_t)row * kD + col;
              const float v = acc[fm][fn][r] * ws;
              const float hv = (EM == E_H_BIAS) ? v + a.bias[col] : *hp + v;
              *hp = hv;
              ss += hv * hv;
            }
          }
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          ss += __shfl_xor(ss, 4);
          ss += __shfl_xor(ss, 8);
          if ((lane & 15) == 0) sSS[wn][rl] = ss;
        } else if constexpr (EM == E_F16_BIAS || EM == E_TIMEIN) {
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn) {
            const int col = cbase + fn * 16 + (lane & 15);
            if (rok && col < N) {
              const float z = acc[fm][fn][r] * ws + a.bias[col];
              a.out16[(size_t)row * a.ldo + col] = (half_t)(EM == E_TIMEIN ? silu(z) : z);
            }
          }
        } else if constexpr (EM == E_QKV) {
          // The wave's 64 columns are one head: Q heads 0..14, K heads 15..19, V heads 20..24.
          const int head = cbase / kHD;
          if (rok && cbase < N) {
            const int b = row / kChunk, ci = row % kChunk;
            const int pos = a.nvalid[b] + ci;
            bf16_t* dst;
            if (head < kHQ) dst = a.q + (((size_t)b * kHQ + head) * kChunk + ci) * kHD;
            else if (head < kHQ + kHKV) dst = a.kc + (((size_t)b * kHKV + head - kHQ) * kChunk + ci) * kHD;
            else dst = a.vc + (((size_t)b * kHKV + head - kHQ - kHKV) * kChunk + ci) * kHD;
#pragma unroll
            for (int fn = 0; fn < 2; ++fn) {
              const int d = fn * 16 + (lane & 15);
              const float x1 = acc[fm][fn][r] * ws, x2 = acc[fm][fn + 2][r] * ws;
              float y1 = x1, y2 = x2;
              if (head < kHQ + kHKV) {  // rotate pairs (d, d + 32)
                const float2 cs = a.rope[pos * (kHD / 2) + d];
                y1 = x1 * cs.x - x2 * cs.y;
                y2 = x1 * cs.y + x2 * cs.x;
              }
              dst[d] = f2bf(y1);
              dst[d + kHD / 2] = f2bf(y2);
            }
          }
        } else if constexpr (EM == E_SWIGLU) {
          // 16-row blocks alternate gate/up: tiles (0,1) and (2,3) are matching pairs.
          if (rok && cbase < N) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const float gt = acc[fm][2 * p][r] * ws, up = acc[fm][2 * p + 1][r] * ws;
              a.out16[(size_t)row * a.ldo + cbase / 2 + p * 16 + (lane & 15)] = (half_t)(silu(gt) * up);
            }
          }
        } else if constexpr (EM == E_ACTOUT) {
#pragma unroll
          for (int fn = 0; fn < T::FN; ++fn) {
            const int col = cbase + fn * 16 + (lane & 15);
            if (rok && col < N) {
              const float v = acc[fm][fn][r] * ws + a.bias[col];
              const size_t xi = (size_t)row * kAD + col;
              const float xn = a.x[xi] + a.dt * v;
              a.x[xi] = xn;
              if (a.vel_out) a.vel_out[xi] = v;
              if (a.st_out) a.st_out[xi] = xn;
              if (a.final_out) a.final_out[xi] = xn;
            }
          }
        }
      }
    }
  }
  if constexpr (EM == E_H_BIAS || EM == E_H_RESID) {
    __syncthreads();
    for (int r = tid; r < T::BM; r += 256) {
      const int row = m0 + r;
      if (row < M) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < T::WN; ++w) s += sSS[w][r];
        a.ss_out[(size_t)row * kSSStride + blockIdx.y] = s;
      }
    }
  }
}

template <class T>
static hipError_t launch_gemm_t(AMode am, EMode em, const GemmArgs& a, hipStream_t s) {
  const dim3 grid((a.M + T::BM - 1) / T::BM, (a.N + T::BN - 1) / T::BN);
  const dim3 block(256);
#define SMOLEXP_GEMM_CASE(AMV, EMV)                                     \
  if (am == AMV && em == EMV) {                                          \
    hipLaunchKernelGGL((gemm_kernel<T, AMV, EMV>), grid, block, 0, s, a); \
    return hipGetLastError();                                            \
  }
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

hipError_t launch_gemm(TileCfg cfg, AMode am, EMode em, const GemmArgs& a, hipStream_t s) {
  if (cfg == T_SKINNY) return launch_gemm_t<SkinnyTile>(am, em, a, s);
  return launch_gemm_t<MedTile>(am, em, a, s);
}

int gemm_ntiles(TileCfg cfg, int N) {
  const int bn = cfg == T_SKINNY ? SkinnyTile::BN : MedTile::BN;
  return (N + bn - 1) / bn;
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
constexpr int kALD = kHD + 8;  // LDS row stride (elements)

template <bool SELF>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[kKB * kALD];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kHD * kALD];
  __shared__ uint8_t sKind[kKB];  // 0 = no key, 1 = valid prefix key, 2 = chunk key

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
  const int nblk = (NK + kKB - 1) / kKB;
  const bf16_t* pk = a.pk + ((size_t)b * kHKV + g) * (size_t)P * kHD;
  const bf16_t* pv = a.pv + ((size_t)b * kHKV + g) * (size_t)P * kHD;
  const bf16_t* ck = SELF ? a.kc + ((size_t)b * kHKV + g) * kChunk * kHD : nullptr;
  const bf16_t* cv = SELF ? a.vc + ((size_t)b * kHKV + g) * kChunk * kHD : nullptr;
  const uint8_t* mk = a.mask + (size_t)b * P;
  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)

  for (int kb = 0; kb < nblk; ++kb) {
    __syncthreads();
    if (tid < kKB) {
      const int j = kb * kKB + tid;
      sKind[tid] = j < P ? (mk[j] ? 1 : 0) : ((SELF && j - P < kChunk) ? 2 : 0);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int v = tid + 256 * it;
      {  // K, row-major: 8 lanes per key row
        const int jl = v >> 3, c = (v & 7) * 8, j = kb * kKB + jl;
        uint4 kv = make_uint4(0, 0, 0, 0);
        if (j < P) {
          if (mk[j]) kv = *reinterpret_cast<const uint4*>(pk + (size_t)j * kHD + c);
        } else if (SELF && j - P < kChunk) {
          kv = *reinterpret_cast<const uint4*>(ck + (size_t)(j - P) * kHD + c);
        }
        *reinterpret_cast<uint4*>(sK + jl * kALD + c) = kv;
      }
      {  // V, stored transposed [d][key]: consecutive lanes take consecutive keys
        const int jl = v & 63, c = (v >> 6) * 8, j = kb * kKB + jl;
        uint4 vv = make_uint4(0, 0, 0, 0);
        if (j < P) {
          if (mk[j]) vv = *reinterpret_cast<const uint4*>(pv + (size_t)j * kHD + c);
        } else if (SELF && j - P < kChunk) {
          vv = *reinterpret_cast<const uint4*>(cv + (size_t)(j - P) * kHD + c);
        }
        const bf16_t* e = reinterpret_cast<const bf16_t*>(&vv);
#pragma unroll
        for (int t = 0; t < 8; ++t) sVt[(c + t) * kALD + jl] = e[t];
      }
    }
    __syncthreads();

    // S^T[key][row] for the 64 keys of the block (4 tiles of 16 keys)
    f32x4 s[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 u = *reinterpret_cast<const uint4*>(sK + (sub * 16 + (lane & 15)) * kALD + kk * 32 + (lane >> 4) * 8);
        s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), qf[kk], s[sub], 0, 0, 0);
      }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jl = sub * 16 + (lane >> 4) * 4 + r;
        const int kind = sKind[jl];
        const bool ok = kind == 1 || (kind == 2 && (kb * kKB + jl - P) <= qi);
        const float val = ok ? s[sub][r] * sl2 : -INFINITY;
        s[sub][r] = val;
        mb = fmaxf(mb, val);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[sub][r] - m_use);
        s[sub][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] *= alpha;

    // O^T[d][row] += V^T[d][key] P^T[key][row], 32 keys per MFMA.  The k-slot
    // order (keys 4q..4q+3 then 16+4q..16+4q+3 for lane group q) is the same
    // for both operands.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[r] = (__bf16)s[2 * h2][r];
        pb[4 + r] = (__bf16)s[2 * h2 + 1][r];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16_t* vp = sVt + (m * 16 + (lane & 15)) * kALD + h2 * 32 + (lane >> 4) * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
        const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), pb, o[m], 0, 0, 0);
      }
    }
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

hipError_t launch_attention(bool self_layer, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(3, kHKV, a.B), block(256);
  if (self_layer) hipLaunchKernelGGL(attn_kernel<true>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(attn_kernel<false>, grid, block, 0, s, a);
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
    // periods geometric from p_min to p_max; evaluated in fp64.
    const int j = blockIdx.x * kTimeRowsPerBlock + (tid >> 4), part = tid & 15;
    const half_t* wr = a.w_t1 + (size_t)j * (2 * kD) + kD;
    for (int k = 0; k < a.n_t; ++k) {
      __syncthreads();
      for (int i = tid; i < kD; i += 256) {
        const int halfd = kD / 2, ii = i % halfd;
        const double frac = (double)ii / (double)(halfd - 1);
        const double period = (double)a.p_min * pow((double)a.p_max / (double)a.p_min, frac);
        const double ang = 2.0 * M_PI * (double)a.t[k] / period;
        se[i] = (float)(i < halfd ? sin(ang) : cos(ang));
      }
      __syncthreads();
      float s = 0.f;
      for (int i = part; i < kD; i += 16) s += (float)wr[i] * se[i];
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
