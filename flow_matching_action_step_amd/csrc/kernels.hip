// HIP kernels of the action-expert denoising loop, written for gfx950 (CDNA4).
//
// GEMMs: C[M,N] = A[M,K] * W[N,K]^T on v_mfma_f32_16x16x32_f16 (fp16
//   operands, fp32 accumulate).  Both operands are stored in 16-row x 8-column
//   micro-tiles (t16_off), so every fragment load and every LDS tile fill
//   reads whole 256-byte runs.  Weights are the
//   checkpoint's bf16 values re-encoded exactly in fp16 with a power-of-two
//   scale per matrix; activations are rounded to fp16 (8x finer than bf16).
//   RMSNorm is fused: its gain is folded into the columns of the weight that
//   follows it (host side); the GEMM multiplies the un-normalised fp16 copy of
//   the residual and scales each finished row by 1/rms(h), whose sum of squares
//   every kernel accumulates on the matrix cores from the A fragments it loads
//   anyway (sumsq_mfma: the diagonal of A A^T).  The A-operand load also fuses
//   the prefix overwrite; epilogues fuse bias, SiLU, RoPE, SwiGLU, the residual
//   add and the Euler update.
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

#include <cstring>
#include <mutex>
#include <type_traits>

namespace smolexp {

typedef half_t f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}

// SiLU(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each):
// the IEEE division sequence would dominate the SwiGLU epilogue.  Large -z gives
// exp2 -> inf, rcp -> 0, result -0; large z gives z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// fp32 values of magnitude 65520 and up (and infinities) round to infinity in fp16.  Each
// thread keeps the largest magnitude it rounds (a running max folds into v_max3 with abs
// modifiers, which ignore NaN: NaN propagates from the inputs as NaN and is not counted) and
// tests it once.
constexpr float kF16Inf = 65520.f;
__device__ __forceinline__ float absmax4(float m, float a, float b, float c, float d) {
  return fmaxf(fmaxf(fmaxf(m, fabsf(a)), fmaxf(fabsf(b), fabsf(c))), fabsf(d));
}

// Report a range overflow seen by this thread (its largest rounded magnitude) to the call's
// status word.
__device__ __forceinline__ void report_range(int* status, float vmax, int bit) {
  if (vmax >= kF16Inf && status) atomicOr(status, bit);
}

// Eight OCP E4M3 weight codes (byte j of c = element j) -> the eight fp16 values they encode,
// exactly (every E4M3 value is an fp16 value), with gfx950's packed conversion (two codes per
// instruction, scale 1).  The fp16 operand passes through unchanged.
typedef half_t f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 w_to_f16x8(const uint4& w) { return w; }
__device__ __forceinline__ uint4 w_to_f16x8(const uint2& c) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.x, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.x, 1.0f, true);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.y, 1.0f, false);
  const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b), __builtin_bit_cast(unsigned, d),
                    __builtin_bit_cast(unsigned, e));
}
// One lane's weight fragment (8 consecutive k of one row): 16 bytes of fp16 or 8 of E4M3.
template <bool W8>
using WFrag = typename std::conditional<W8, uint2, uint4>::type;
// The load is issued unconditionally (from offset 0 when !ok, inside the buffer) and zeroed
// afterwards: a load under a branch made the compiler wait for it before issuing the next
// ones (a register copy out of the branch), serializing the round trips.
// UNCOND = false keeps the conditional form (for kernels whose loads were already issued
// together, where the selects only add instructions).
template <bool W8, bool UNCOND = true>
__device__ __forceinline__ WFrag<W8> load_wfrag(const half_t* W, size_t off, bool ok) {
  if constexpr (W8) {
    const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(W) + (ok ? off : 0));
    return make_uint2(ok ? v.x : 0u, ok ? v.y : 0u);
  } else if constexpr (UNCOND) {
    const uint4 v = *reinterpret_cast<const uint4*>(W + (ok ? off : 0));
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
  } else {
    return ok ? *reinterpret_cast<const uint4*>(W + off) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint4 pack8(const float* v) {
  union { half_t h[8]; uint4 u; } p;
#pragma unroll
  for (int e = 0; e < 8; ++e) p.h[e] = (half_t)v[e];
  return p.u;
}

// ----------------------------------------------------------------------------
// GEMM
// ----------------------------------------------------------------------------
// Three kernels share the A-operand loaders and the epilogues (plan_for picks one per
// projection and row count):
//  * gemm_skinny (one query at batch 1; up to a few thousand rows for the narrow
//    products): one 512-thread workgroup per 1, 2 or 4 16-column blocks and 1, 2 or 4
//    16-row blocks.  Its 8 waves split K; each wave issues every load it needs (its
//    weight fragments and A fragments) at once, so the kernel waits for memory about
//    once, then the waves' partial tiles meet in LDS.
//  * gemm_tiled: 64/128 x 128 output tiles, four waves, BK = 64 slabs
//    double-buffered in LDS through registers (the time MLP at large row counts).
//  * gemm_big (K a multiple of its 32- or 64-column slab): 64 or 128 x 128 tiles, eight waves, an LDS ring
//    filled by direct global->LDS loads.
// Epilogues run on the finished fp32 tile, staged in LDS or (the residual projections)
// taken from the waves' partials or accumulators.
//
// Weight row order inside each 16-row block (set by the host when it loads
// the weights) keeps every pair an epilogue needs in one block:
//  * Q and K heads: block q of a head holds dims q*8..q*8+7, then 32+q*8..
//    32+q*8+7, so column e pairs with e+8 for the rotation of (d, d+32);
//  * gate/up: block j holds gate rows 8j..8j+7, then up rows 8j..8j+7;
//  * V heads and every other matrix keep their natural order.

// Eight consecutive A elements of row `row`, columns k..k+7, converted to the
// fp16 MFMA operand (ok = inside the matrix; otherwise zeros).
// UNCOND (fp16 operands): issue the load for every lane (element 0 when !ok) and zero it
// afterwards, with no branch around the load (see load_wfrag).
template <int AM, bool UNCOND = false>
__device__ __forceinline__ uint4 load_a8(const GemmArgs& a, int row, int k, bool ok, float rscale,
                                         bool write_x, float& vmax) {
  (void)rscale;
  if constexpr ((AM == A_F16 || AM == A_NORM) && UNCOND) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const half_t*>(a.A) + (ok ? t16_off(row, k, a.lda >> 3) : 0));
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
  } else if constexpr (AM == A_F16 || AM == A_NORM) {
    return ok ? *reinterpret_cast<const uint4*>(static_cast<const half_t*>(a.A) + t16_off(row, k, a.lda >> 3))
              : make_uint4(0, 0, 0, 0);
  } else {  // A_X: Euler state; rows i < ow_rows of each chunk take the flow-path point t*eps + (1-t)*prev
    // Every lane loads its state row (row 0 past the end); with an overwrite (a uniform
    // kernel argument) also the noise and previous-chunk rows (row 0 where not overwritten);
    // the values are selected after all loads are issued, with no branch around a load.
    const float* xs = static_cast<const float*>(a.A) + (size_t)(ok ? row : 0) * a.lda + k;
    const float4 x0 = *reinterpret_cast<const float4*>(xs), x1 = *reinterpret_cast<const float4*>(xs + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (a.ow_rows > 0) {
      const int ci = row % kChunk, b = row / kChunk;
      const bool ow = ok && ci < a.ow_rows;
      const float* ep = a.noise + (size_t)(ow ? row : 0) * kAD + k;
      const float* pp = a.prev + ((size_t)(ow ? b : 0) * a.ow_rows + (ow ? ci : 0)) * kAD + k;
      const float4 e0 = *reinterpret_cast<const float4*>(ep), e1 = *reinterpret_cast<const float4*>(ep + 4);
      const float4 p0 = *reinterpret_cast<const float4*>(pp), p1 = *reinterpret_cast<const float4*>(pp + 4);
      const float t = a.t, u = 1.0f - a.t;
      const float w[8] = {t * e0.x + u * p0.x, t * e0.y + u * p0.y, t * e0.z + u * p0.z, t * e0.w + u * p0.w,
                          t * e1.x + u * p1.x, t * e1.y + u * p1.y, t * e1.z + u * p1.z, t * e1.w + u * p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = ow ? w[e] : v[e];
      if (ow && write_x) {  // one workgroup column stores the overwritten rows into the state
        float* xp = a.x + (size_t)row * kAD + k;
        *reinterpret_cast<float4*>(xp) = make_float4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<float4*>(xp + 4) = make_float4(w[4], w[5], w[6], w[7]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ok ? v[e] : 0.f;
    vmax = absmax4(absmax4(vmax, v[0], v[1], v[2], v[3]), v[4], v[5], v[6], v[7]);
    return pack8(v);
  }
}

// Row sums of squares on the matrix cores: with one A fragment (16 rows x 32 k)
// as both operands the MFMA accumulates A A^T, whose diagonal holds the sum of
// squares of each row (fp16 products are exact in fp32).  One MFMA per 16 rows
// per k-step, far cheaper than VALU dot products interleaved with the GEMM.
__device__ __forceinline__ f32x4 sumsq_mfma(const f16x8& af, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(af, af, acc, 0, 0, 0);
}
// Row m (0..15) of a 16-row tile has its diagonal element in lane 16 (m / 4) + m,
// register m % 4; every lane reads the one for row 4 (lane / 16) + r (the rows
// whose accumulators it holds in register r).
__device__ __forceinline__ float diag_for_row(const f32x4& sq, int r, int lane) {
  return __shfl(sq[r], 20 * (lane >> 4) + r);
}

// 1/rms of a row from its sum of squares.
__device__ __forceinline__ float rms_scale_qk(float inv_k, float eps, float sumsq) { return rsqrtf(sumsq * inv_k + eps); }
__device__ __forceinline__ float rms_scale(const GemmArgs& a, float sumsq) { return rms_scale_qk(a.inv_k, a.eps, sumsq); }

// Epilogue on a finished tile sC[BM][LDC] (fp32, weight and row scales
// applied) whose rows start at m0 and columns at n0 (BN a multiple of 16).
// The blocked outputs (fp16 activations, the fp32 residual and its fp16 copy)
// are written with 16 consecutive lanes on 16 consecutive rows of one column
// chunk, i.e. contiguous runs of 256 (128) bytes per store.
// PRE: the global inputs of the thread's units were loaded at kernel start into
// pre[] (E_QKV, one unit per thread: the 16 cos/sin values of a rotated block;
// E_H_RESID, one row block per wave: the residual values of chunk t in pre[t],
// BN / 16 of them).
// Column chunks of the fp32 residual (t32_off) and of its fp16 copy (t16_off) by epilogue:
// the expert's 720 (its copy stored over 768 columns), or the prefix model's 960.
__host__ __device__ constexpr int resid_k4(int em) { return em == E_PF_RESID ? kLmD / 4 : kD / 4; }
__host__ __device__ constexpr int resid16_kc(int em) { return em == E_PF_RESID ? kLmD / 8 : kKPad / 8; }

// Store of a 4-, 8- or 16-byte value, nontemporal when NTS.
template <bool NTS, typename T>
__device__ __forceinline__ void st_out(T* p, const T& v) {
  if constexpr (NTS) {
    typedef unsigned V __attribute__((ext_vector_type(sizeof(T) / 4)));
    __builtin_nontemporal_store(__builtin_bit_cast(V, v), reinterpret_cast<V*>(p));
  } else {
    *p = v;
  }
}

template <int EM, int BM, int BN, int LDC, int NT, bool PRE = false, bool NTS = false>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const float* sC, int m0, int n0,
                                              const float4* pre = nullptr) {
  constexpr int NB = BN / 16, UPR = NB * 8;
  static_assert(UPR <= 64 && 64 % UPR == 0, "rows inside one wave");
  static_assert(!PRE || (EM != E_QKV && EM != E_PF_QKV) || (BM * NB <= NT && NB <= 4), "PRE: one E_QKV unit per thread");
  static_assert(!PRE || (EM != E_H_RESID && EM != E_PF_RESID) || BM / 16 <= NT / 64,
                "PRE: one E_H_RESID row block per wave");
  const int M = a.M, N = a.N;
  if constexpr (EM == E_QKV || EM == E_PF_QKV) {
    // Work unit = (row, 16-column block): the block is 8 rotation pairs of one Q/K
    // head (dims q*8.. and 32+q*8.., one 16-byte run each) or 16 consecutive V dims.
    for (int g = threadIdx.x; g < BM * NB; g += NT) {
      const int r = g / NB, blk = g % NB;
      const int row = m0 + r, cb = n0 + blk * 16;
      if (row >= M || cb >= N) continue;
      const float4* src = reinterpret_cast<const float4*>(sC + r * LDC + blk * 16);
      const float4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
      const float v1[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float v2[8] = {c2.x, c2.y, c2.z, c2.w, c3.x, c3.y, c3.z, c3.w};
      const int seq = EM == E_PF_QKV ? a.seq : kChunk;  // rows per query
      const int head = cb / kHD, b = row / seq, ci = row % seq;
      (void)pre;
      bf16_t* dst;
      if (head < kHQ) dst = a.q + (((size_t)b * kHQ + head) * seq + ci) * kHD;
      else if (head < kHQ + kHKV) dst = a.kc + (((size_t)b * kHKV + head - kHQ) * seq + ci) * kHD;
      else dst = a.vc + (((size_t)b * kHKV + head - kHQ - kHKV) * seq + ci) * kHD;
      union { bf16_t e[8]; uint4 u; } lo, hi;
      if (head < kHQ + kHKV) {  // rotate the pairs (d, d + 32), d = d0..d0+7, at this row's position
        const int d0 = ((cb % kHD) / 16) * 8;
        float4 q0, q1, q2, q3;
        if constexpr (PRE) {
          q0 = pre[0]; q1 = pre[1]; q2 = pre[2]; q3 = pre[3];
        } else {
          const float4* cs4 = reinterpret_cast<const float4*>(a.ropeq + (size_t)row * (kHD / 2) + d0);
          q0 = cs4[0]; q1 = cs4[1]; q2 = cs4[2]; q3 = cs4[3];
        }
        const float cs[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                              q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = cs[2 * e], sn = cs[2 * e + 1];
          lo.e[e] = f2bf(v1[e] * c - v2[e] * sn);
          hi.e[e] = f2bf(v1[e] * sn + v2[e] * c);
        }
        st_out<NTS>(reinterpret_cast<uint4*>(dst + d0), lo.u);
        st_out<NTS>(reinterpret_cast<uint4*>(dst + d0 + kHD / 2), hi.u);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo.e[e] = f2bf(v1[e]);
          hi.e[e] = f2bf(v2[e]);
        }
        st_out<NTS>(reinterpret_cast<uint4*>(dst + cb % kHD), lo.u);
        st_out<NTS>(reinterpret_cast<uint4*>(dst + cb % kHD + 8), hi.u);
      }
    }
    return;
  }
  if constexpr (EM == E_SWIGLU || EM == E_TIMEIN) {
    // Work unit = (row, one 8-column chunk of the fp16 output).  SwiGLU: the
    // 16-column block c of the tile holds gate (8) then up (8) of output chunk c.
    constexpr int NC = EM == E_SWIGLU ? BN / 16 : BN / 8;  // output chunks per tile row
    const int kco = a.ldo >> 3;
    float vmax = 0.f;
    for (int g = threadIdx.x; g < BM * NC; g += NT) {
      const int r = (g & 15) + 16 * ((g >> 4) / NC), c = (g >> 4) % NC;
      const int row = m0 + r;
      float v[8];
      int col;
      if constexpr (EM == E_SWIGLU) {
        if (row >= M || n0 + c * 16 >= N) continue;
        col = (n0 + c * 16) / 2;
        const float4* p = reinterpret_cast<const float4*>(sC + r * LDC + c * 16);
        const float4 g0 = p[0], g1 = p[1], u0 = p[2], u1 = p[3];
        const float gt[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float up[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = silu(gt[e]) * up[e];
      } else {
        col = n0 + c * 8;
        if (row >= M || col >= N) continue;
        const float4* p = reinterpret_cast<const float4*>(sC + r * LDC + c * 8);
        const float4* bp = reinterpret_cast<const float4*>(a.bias + col);
        const float4 a0 = p[0], a1 = p[1], b0 = bp[0], b1 = bp[1];
        const float z[8] = {a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w,
                            a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = silu(z[e]);
      }
      vmax = absmax4(absmax4(vmax, v[0], v[1], v[2], v[3]), v[4], v[5], v[6], v[7]);
      st_out<NTS>(reinterpret_cast<uint4*>(a.out16 + t16_off(row, col, kco)), pack8(v));
    }
    report_range(a.status, vmax, EM == E_SWIGLU ? kRangeFfn : kRangeTime);
    return;
  }
  if constexpr (EM == E_H_BIAS || EM == E_H_RESID || EM == E_PF_RESID) {
    // Work unit = (row, one 4-column chunk of the fp32 residual and of its fp16 copy).
    // Lane = r16 + 16 * part: a wave owns one 16-row block per pass and its four parts
    // take every fourth chunk.
    constexpr int NC4 = BN / 4, NWV = NT / 64, RB = BM / 16;
    static_assert(NC4 % 4 == 0 && NT % 64 == 0, "uniform trip counts");
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15, part = lane >> 4;
    float vmax = 0.f;
    for (int rb = wv; rb < RB; rb += NWV) {
      const int r = rb * 16 + r16, row = m0 + r;
      const bool live = row < M;
#pragma unroll
      for (int t = 0; t < NC4 / 4; ++t) {
        const int c = part + 4 * t, col = n0 + c * 4;
        if (live && col < N) {
          const float4 v = *reinterpret_cast<const float4*>(sC + r * LDC + c * 4);
          float4* hp = reinterpret_cast<float4*>(a.h + t32_off(row, col, resid_k4(EM)));
          float4 o;
          if constexpr (EM == E_H_BIAS) {
            const float4 b = *reinterpret_cast<const float4*>(a.bias + col);
            o = make_float4(v.x + b.x, v.y + b.y, v.z + b.z, v.w + b.w);
          } else {
            const float4 hv = PRE ? pre[t] : *hp;
            o = make_float4(hv.x + v.x, hv.y + v.y, hv.z + v.z, hv.w + v.w);
          }
          st_out<NTS>(hp, o);
          vmax = absmax4(vmax, o.x, o.y, o.z, o.w);
          union { half_t e[4]; uint2 u; } o16;
          o16.e[0] = (half_t)o.x; o16.e[1] = (half_t)o.y; o16.e[2] = (half_t)o.z; o16.e[3] = (half_t)o.w;
          st_out<NTS>(reinterpret_cast<uint2*>(a.h16 + t16_off(row, col, resid16_kc(EM))), o16.u);
        }
      }
    }
    report_range(a.status, vmax, kRangeResidual);
    return;
  }
  if constexpr (EM == E_ACTOUT) {
    // action_out + Euler update on the row-major state.  Work unit = (row,
    // 16-column block, e < 8) covering columns e and e + 8 of the block.
    for (int g = threadIdx.x; g < BM * UPR; g += NT) {
      const int r = g / UPR, blk = (g % UPR) / 8, e = g % 8;
      const int row = m0 + r, cb = n0 + blk * 16;
      if (row >= M || cb >= N) continue;
      const float v1 = sC[r * LDC + blk * 16 + e], v2 = sC[r * LDC + blk * 16 + 8 + e];
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
}

// A workgroup computes CB 16-column blocks for RB 16-row blocks (rows m0 .. m0 + 16 RB - 1);
// wave w takes k-steps w*KPW .. w*KPW+KPW-1 (32 wide each), so every fragment of the
// product stays in registers (K <= 8 x KPW x 32).  What bounds these launches is the bytes
// one workgroup streams through its CU (its A rows and weight rows), so the rows are split
// over row tiles of 16 RB rows per column-block group.  The row tiles of one group sit on one
// XCD (workgroup i runs on XCD i % 8), so that XCD's L2 fetches those weight rows once.  A_NORM: the rows of fp16(h) go to the
// MFMA unscaled, so no load waits on the row scale; each wave also sums the
// squares of its slice of every row, and 1/rms(row) scales the finished sums
// (a per-row constant, so this equals normalising first up to rounding).
// W8: the weights are E4M3 codes (8 bytes per lane and k-step, widened to fp16 in registers)
// and each output column n is scaled by its row scale wrs[n] instead of w_scale.
template <int AM, int EM, int KPW, int RB, int CB = 1, bool W8 = false>
__global__ __launch_bounds__(512) void gemm_skinny(const GemmArgs a) {
  constexpr int NW = 8, BM = 16 * RB, BN = 16 * CB, LDC = BN;
  static_assert(RB == 1 || RB == 2 || RB == 4, "row blocks per workgroup");
  static_assert(CB == 1 || CB == 2 || CB == 4, "column blocks per workgroup");
  constexpr bool PRE = EM == E_QKV || EM == E_PF_QKV || EM == E_H_RESID || EM == E_PF_RESID;
  __shared__ float sRed[NW * BM * BN];
  __shared__ float sC[BM * LDC];
  __shared__ float sQ[AM == A_NORM ? NW : 1][BM];  // per-wave partial sums of squares of the rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = a.M, N = a.N, K = a.K;
  // workgroup -> (column block group, row tile): the row tiles of one group are consecutive
  // in j and share XCD = blockIdx.x % 8 = group % 8
  const int nrt = (M + BM - 1) / BM;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int nb = xcd + 8 * (j / nrt), m0 = (j % nrt) * BM;
  const int n0 = nb * BN;
  if (n0 >= N) return;  // grid padded to whole XCD rounds; no barrier before this
  const int nks = (K + 31) / 32;
  const int kl = (lane >> 4) * 8;

  // epilogue inputs, loaded with the operands, in epilogue_tile's unit mapping: E_QKV thread
  // g < BM * CB owns row m0 + g / CB, column block g % CB; E_H_RESID lane r + 16 p of wave
  // w < RB owns row m0 + 16 w + r, columns n0 + 4 (p + 4 t).. for t < CB
  // Rows or columns past the end load from row 0 / column 0, which exist; the epilogue reads
  // only the units it owns.  No branch inside a wave around the loads: one made the compiler
  // wait for them before issuing the operand loads.
  float4 pre[4];
  if constexpr (EM == E_QKV || EM == E_PF_QKV) {
    if (w < (BM * CB + 63) / 64) {  // the waves that own units (uniform per wave)
      const int g = tid < BM * CB ? tid : 0;
      const int row = m0 + g / CB, cb0 = n0 + (g % CB) * 16;
      const int d0 = ((cb0 % kHD) / 16) * 8;
      const float4* cs4 = reinterpret_cast<const float4*>(a.ropeq + (size_t)(row < M ? row : 0) * (kHD / 2) + d0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pre[jj] = cs4[jj];
    }
  } else if constexpr (EM == E_H_RESID || EM == E_PF_RESID) {
    const int row = m0 + w * 16 + (lane & 15);
    const bool rok = w < RB && row < M;
#pragma unroll
    for (int t = 0; t < CB; ++t) {
      const int col = n0 + ((lane >> 4) + 4 * t) * 4;
      const bool ok = rok && col < N;
      pre[t] = *reinterpret_cast<const float4*>(a.h + (ok ? t32_off(row, col, resid_k4(EM)) : 0));
    }
  }
  // the weight scale of the one output column this thread reduces (BN divides 512)
  static_assert(512 % BN == 0, "one reduction column per thread");
  float wsc = a.w_scale;
  if constexpr (W8) {  // loaded unconditionally (a clamped index), as load_wfrag does
    const int col = n0 + tid % BN;
    const float v = a.wrs[col < N ? col : N - 1];
    wsc = col < N ? v : 0.f;
  }
  // gate/up (fp16) issues its loads together in either form and runs faster with the
  // conditional one (4.25 against 4.35 us per launch at batch 1); the others need the
  // branch-free form (see load_wfrag)
  constexpr bool UNC = W8 || EM != E_SWIGLU;
  WFrag<W8> wf[KPW][CB];
  uint4 af[KPW][RB];
  float xmax = 0.f;  // A_X: the largest magnitude of the Euler state rounded to fp16
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = w * KPW + i, k = ks * 32 + kl;
    const bool kok = ks < nks && k < K;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = n0 + cb * 16 + (lane & 15);
      wf[i][cb] = load_wfrag<W8, UNC>(a.W, t16_off(n, k, a.ldw >> 3), kok && n < N);
    }
#pragma unroll
    for (int fm = 0; fm < RB; ++fm) {
      const int row = m0 + fm * 16 + (lane & 15);
      const bool ok = kok && row < M;
      af[i][fm] = load_a8<AM, UNC>(a, row, k, ok, 1.f, nb == 0, xmax);
    }
  }
  // the residual modes finish in the waves that own the units (below): their bias and (8-bit
  // weights) the row scales of their four columns, issued after the operands (the youngest
  // loads; only the epilogue waits for them)
  constexpr bool FUSED = EM == E_H_RESID || EM == E_H_BIAS || EM == E_PF_RESID;
  float4 bias4[FUSED ? CB : 1], wsc4[FUSED ? CB : 1];
  if constexpr (FUSED) {
#pragma unroll
    for (int t = 0; t < CB; ++t) {
      const int col = n0 + ((lane >> 4) + 4 * t) * 4, cc = col < N ? col : 0;
      if constexpr (EM == E_H_BIAS) bias4[t] = *reinterpret_cast<const float4*>(a.bias + cc);
      if constexpr (W8) wsc4[t] = *reinterpret_cast<const float4*>(a.wrs + cc);
      else wsc4[t] = make_float4(a.w_scale, a.w_scale, a.w_scale, a.w_scale);
    }
  }
  f32x4 acc[RB][CB];
#pragma unroll
  for (int fm = 0; fm < RB; ++fm)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[fm][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const f16x8 bw = __builtin_bit_cast(f16x8, w_to_f16x8(wf[i][cb]));
#pragma unroll
      for (int fm = 0; fm < RB; ++fm)
        acc[fm][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af[i][fm]), bw, acc[fm][cb], 0, 0, 0);
    }
  }
  if constexpr (AM == A_NORM) {
    // this wave's share of each row's sum of squares, from the diagonal of A A^T over its K slice
#pragma unroll
    for (int fm = 0; fm < RB; ++fm) {
      f32x4 sq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KPW; ++i) sq = sumsq_mfma(__builtin_bit_cast(f16x8, af[i][fm]), sq);
      if (((lane & 15) >> 2) == (lane >> 4)) sQ[w][fm * 16 + (lane & 15)] = sq[lane & 3];
    }
  }
#pragma unroll
  for (int fm = 0; fm < RB; ++fm)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sRed[(w * BM + fm * 16 + (lane >> 4) * 4 + r) * BN + cb * 16 + (lane & 15)] = acc[fm][cb][r];
  __syncthreads();
  if constexpr (FUSED) {
    // Residual modes: lane r16 + 16 p of wave w < RB sums its 16-byte units (row m0 + 16 w + r16,
    // columns n0 + 4 (p + 4 t) .. + 3) straight from the waves' partials, in the same order as
    // the tile reduction below, and applies the epilogue: no second LDS tile, one barrier fewer.
    const int r16 = lane & 15, part = lane >> 4;
    float vmax = 0.f;
    if (w < RB) {
      const int r = w * 16 + r16, row = m0 + r;
#pragma unroll
      for (int t = 0; t < CB; ++t) {
        const int c = part + 4 * t, col = n0 + c * 4;
        if (row < M && col < N) {
          float4 sm = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) {
            const float4 pv = *reinterpret_cast<const float4*>(sRed + (w2 * BM + r) * BN + c * 4);
            sm.x += pv.x; sm.y += pv.y; sm.z += pv.z; sm.w += pv.w;
          }
          const float4 v = make_float4(sm.x * wsc4[t].x, sm.y * wsc4[t].y, sm.z * wsc4[t].z, sm.w * wsc4[t].w);
          float4* hp = reinterpret_cast<float4*>(a.h + t32_off(row, col, resid_k4(EM)));
          float4 o;
          if constexpr (EM == E_H_BIAS) {
            o = make_float4(v.x + bias4[t].x, v.y + bias4[t].y, v.z + bias4[t].z, v.w + bias4[t].w);
          } else {
            const float4 hv = PRE ? pre[t] : *hp;
            o = make_float4(hv.x + v.x, hv.y + v.y, hv.z + v.z, hv.w + v.w);
          }
          *hp = o;
          vmax = absmax4(vmax, o.x, o.y, o.z, o.w);
          union { half_t e[4]; uint2 u; } o16;
          o16.e[0] = (half_t)o.x; o16.e[1] = (half_t)o.y; o16.e[2] = (half_t)o.z; o16.e[3] = (half_t)o.w;
          *reinterpret_cast<uint2*>(a.h16 + t16_off(row, col, resid16_kc(EM))) = o16.u;
        }
      }
    }
    report_range(a.status, vmax, kRangeResidual);
    return;
  }
  for (int i = tid; i < BM * BN; i += 512) {
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) s += sRed[w2 * BM * BN + i];
    float sc = wsc;
    if constexpr (AM == A_NORM) {  // RMSNorm: rows were multiplied unscaled, 1/rms(h) applied here
      float q = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) q += sQ[w2][i / BN];
      sc *= rms_scale(a, q);
    }
    sC[i] = s * sc;
  }
  __syncthreads();
  if constexpr (AM == A_X) report_range(a.status, xmax, kRangeTime);
  epilogue_tile<EM, BM, BN, LDC, 512, PRE>(a, sC, m0, n0, pre);
}

// ----------------------------------------------------------------------------
// Step boundary: the final RMSNorm + action_out + Euler update of step k, then the prefix
// overwrite and the time MLP's first layer (action_in folded in) of step k + 1
// ----------------------------------------------------------------------------
// Both halves are row-local: an action row needs one row of fp16(h) and the whole of
// action_out's weights, and the next step's time-MLP row needs that action row and the whole
// [720][32] matrix.  A workgroup of eight waves takes 16 rows and one of G groups of the time
// MLP's 45 column tiles: the waves split action_out's K as gemm_skinny does (three k-steps
// each, both 16-column blocks; the G workgroups of a row block repeat this small product), the
// partial sums meet in LDS, one thread per (row, action column) finishes the Euler update and
// the overwrite (group 0 stores the state and the records), and the waves then multiply the 16
// updated rows by the group's column tiles (K = 32, one MFMA per tile).  The state of step k
// is read from v.x and that of step k + 1 written to t.x, another buffer, since every
// workgroup of a row block reads the old state.  Every sum is formed from the same operands in the same order as
// in the two separate launches (action_out, then time_in), so the results are the same bits.
// v: action_out's arguments (A_NORM operand h16, bias, x, dt, records); t: the next step's
// time_in arguments (its flow time, time vector, overwrite rows, output s16).
// TOUT (one query's 50 rows): the time MLP's second layer too (o: time_out's arguments, the
// residual stream h0 = W_t2 s + b_t2 and its fp16 copy).  Workgroup (row block, c) then computes
// all 45 column tiles of the hidden layer s into LDS and the 16 output columns 16 c .. of the
// second layer from them, as gemm_skinny<A_F16, E_H_BIAS, 3, 1, 1> would from the stored s (same
// k-steps per wave, same order of the partial sums, same epilogue), so again the same bits.
struct BoundaryArgs {
  GemmArgs v, t, o;
};

// a * b + c with the product rounded before the sum (no fused multiply-add), as when the product
// is stored and the sum formed later
__device__ __forceinline__ float mul_add_rounded(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b + c;
}

template <bool W8, bool TOUT = false>
__global__ __launch_bounds__(512) void step_boundary_kernel(const BoundaryArgs ba) {
  constexpr int NW = 8, KPW = 3, NCB = kAD / 16, NTT = kD / 16, TPW = (NTT + NW - 1) / NW;
  static_assert(NCB * 16 == kAD && NTT * 16 == kD && 16 * kAD == 512, "one (row, action column) per thread");
  const GemmArgs& a = ba.v;
  const GemmArgs& t = ba.t;
  __shared__ float sRed[NW * 16 * kAD];
  __shared__ float sQ[NW][16];
  __shared__ __attribute__((aligned(16))) float sX[16][kAD];
  __shared__ __attribute__((aligned(16))) half_t sZ[16][kD];
  __shared__ __attribute__((aligned(16))) float sRedO[TOUT ? NW * 16 * 16 : 1];  // TOUT: the waves' partial tiles
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // G workgroups per row block: the hidden layer's column groups, or (TOUT) the second layer's
  // 16-column blocks, each with the whole hidden layer
  const int G = gridDim.x / ((a.M + 15) / 16), rb = blockIdx.x / G, cg = blockIdx.x % G;
  const int M = a.M, K = a.K, m0 = rb * 16;
  const int nks = (K + 31) / 32, kl = (lane >> 4) * 8;
  const int t_lo = TOUT ? 0 : cg * NTT / G, t_hi = TOUT ? NTT : (cg + 1) * NTT / G;  // hidden-layer column tiles

  // every load first: action_out's operands (as gemm_skinny<A_NORM, E_ACTOUT, 3, 1, 2>), the time
  // MLP's weight fragments and time-vector entries of this wave's column tiles, the thread's
  // Euler-update inputs and its overwrite inputs (unconditional, clamped to row 0)
  WFrag<W8> wf[KPW][NCB];
  uint4 af[KPW];
  float unused_max = 0.f;
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int ks = w * KPW + i, k = ks * 32 + kl;
    const bool kok = ks < nks && k < K;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      wf[i][cb] = load_wfrag<W8, true>(a.W, t16_off(cb * 16 + (lane & 15), k, a.ldw >> 3), kok);
    const int row = m0 + (lane & 15);
    af[i] = load_a8<A_NORM, true>(a, row, k, kok && row < M, 1.f, false, unused_max);
  }
  WFrag<W8> wt[TPW];
  float tb[TPW], ts[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int n = t_lo + w + NW * i, col = (n < t_hi ? n : 0) * 16 + (lane & 15);
    wt[i] = load_wfrag<W8, true>(t.W, t16_off(col, kl, t.ldw >> 3), n < t_hi);
    tb[i] = t.bias[col];
    ts[i] = W8 ? t.wrs[col] : t.w_scale;
  }
  // TOUT: the second layer's weight fragments of this wave's k-steps (16 rows of column block cg)
  // and, for wave 0 (which finishes the tile), its bias and weight scales
  const GemmArgs& go = ba.o;
  WFrag<W8> wo[TOUT ? KPW : 1];
  float4 bias4 = make_float4(0.f, 0.f, 0.f, 0.f), wsc4 = bias4;
  if constexpr (TOUT) {
    const int nksO = (go.K + 31) / 32;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int ks = w * KPW + i, k = ks * 32 + kl;
      wo[i] = load_wfrag<W8, true>(go.W, t16_off(cg * 16 + (lane & 15), k, go.ldw >> 3), ks < nksO && k < go.K);
    }
    const int col = cg * 16 + (lane >> 4) * 4;
    bias4 = *reinterpret_cast<const float4*>(go.bias + col);
    if constexpr (W8) wsc4 = *reinterpret_cast<const float4*>(go.wrs + col);
    else wsc4 = make_float4(go.w_scale, go.w_scale, go.w_scale, go.w_scale);
  }
  const int r = tid / kAD, c = tid % kAD, row = m0 + r;
  const bool rok = row < M;
  const size_t xi = (size_t)(rok ? row : 0) * kAD + c;
  const float xold = a.x[xi], bo = a.bias[c], vsc = W8 ? a.wrs[c] : a.w_scale;
  const int ci = row % kChunk, bq = row / kChunk;
  const bool ow = rok && ci < t.ow_rows;
  float e_ow = 0.f, p_ow = 0.f;
  if (t.ow_rows > 0) {  // uniform kernel argument
    e_ow = t.noise[(size_t)(ow ? row : 0) * kAD + c];
    p_ow = t.prev[((size_t)(ow ? bq : 0) * t.ow_rows + (ow ? ci : 0)) * kAD + c];
  }

  // action_out: this wave's K slice of both column blocks, and of each row's sum of squares
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 sq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af[i]),
                                                       __builtin_bit_cast(f16x8, w_to_f16x8(wf[i][cb])), acc[cb], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < KPW; ++i) sq = sumsq_mfma(__builtin_bit_cast(f16x8, af[i]), sq);
  if (((lane & 15) >> 2) == (lane >> 4)) sQ[w][lane & 15] = sq[lane & 3];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sRed[(w * 16 + (lane >> 4) * 4 + rr) * kAD + cb * 16 + (lane & 15)] = acc[cb][rr];
  __syncthreads();

  // thread (r, c): the velocity, the Euler step, the records, then the next step's overwrite
  {
    float sm = 0.f, q = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) sm += sRed[(w2 * 16 + r) * kAD + c];
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) q += sQ[w2][r];
    const float u = mul_add_rounded(sm, vsc * rms_scale(a, q), bo);
    const float x1 = xold + a.dt * u;
    const float tt = t.t, om = 1.0f - t.t;
    const float xn = ow ? __builtin_fmaf(tt, e_ow, om * p_ow) : x1;  // t eps + (1 - t) prev, as time_in forms it
    if (rok && cg == 0) {
      t.x[xi] = xn;
      if (a.vel_out) a.vel_out[xi] = u;
      if (a.st_out) a.st_out[xi] = x1;
    }
    sX[r][c] = rok ? xn : 0.f;
  }
  __syncthreads();

  // time MLP, first layer: z = SiLU(W x + time vector) for this wave's column tiles
  float v8[8];
  {
    const float4 x0 = *reinterpret_cast<const float4*>(&sX[lane & 15][kl]);
    const float4 x4 = *reinterpret_cast<const float4*>(&sX[lane & 15][kl + 4]);
    v8[0] = x0.x; v8[1] = x0.y; v8[2] = x0.z; v8[3] = x0.w; v8[4] = x4.x; v8[5] = x4.y; v8[6] = x4.z; v8[7] = x4.w;
  }
  const float xmax = absmax4(absmax4(0.f, v8[0], v8[1], v8[2], v8[3]), v8[4], v8[5], v8[6], v8[7]);
  const f16x8 xa = __builtin_bit_cast(f16x8, pack8(v8));
  float zmax = 0.f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int n = t_lo + w + NW * i;
    if (n >= t_hi) break;  // uniform per wave
    const f32x4 z = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, __builtin_bit_cast(f16x8, w_to_f16x8(wt[i])),
                                                           f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float sv = silu(mul_add_rounded(z[rr], ts[i], tb[i]));
      zmax = fmaxf(zmax, fabsf(sv));
      sZ[(lane >> 4) * 4 + rr][n * 16 + (lane & 15)] = (half_t)sv;
    }
  }
  report_range(t.status, fmaxf(xmax, zmax), kRangeTime);
  __syncthreads();
  if constexpr (TOUT) {
    // the second layer: this wave's three k-steps of the hidden layer (from LDS) against the
    // weight fragments, the partial tiles summed in wave order, bias added, h0 and fp16(h0) stored
    const int nksO = (go.K + 31) / 32;
    f32x4 acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int ks = w * KPW + i, k = ks * 32 + kl;
      const bool kok = ks < nksO && k < go.K;
      const uint4 zf = kok ? *reinterpret_cast<const uint4*>(&sZ[lane & 15][k]) : make_uint4(0, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, zf),
                                                    __builtin_bit_cast(f16x8, w_to_f16x8(wo[i])), acc2, 0, 0, 0);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sRedO[(w * 16 + (lane >> 4) * 4 + rr) * 16 + (lane & 15)] = acc2[rr];
    __syncthreads();
    if (w == 0) {
      const int r16 = lane & 15, part = lane >> 4, orow = m0 + r16, col = cg * 16 + part * 4;
      float vmax = 0.f;
      if (orow < M && col < go.N) {
        float4 sm = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          const float4 pv = *reinterpret_cast<const float4*>(sRedO + (w2 * 16 + r16) * 16 + part * 4);
          sm.x += pv.x; sm.y += pv.y; sm.z += pv.z; sm.w += pv.w;
        }
        const float4 v = make_float4(sm.x * wsc4.x, sm.y * wsc4.y, sm.z * wsc4.z, sm.w * wsc4.w);
        const float4 o = make_float4(v.x + bias4.x, v.y + bias4.y, v.z + bias4.z, v.w + bias4.w);
        *reinterpret_cast<float4*>(go.h + t32_off(orow, col, kD / 4)) = o;
        vmax = absmax4(vmax, o.x, o.y, o.z, o.w);
        union { half_t e[4]; uint2 u; } o16;
        o16.e[0] = (half_t)o.x; o16.e[1] = (half_t)o.y; o16.e[2] = (half_t)o.z; o16.e[3] = (half_t)o.w;
        *reinterpret_cast<uint2*>(go.h16 + t16_off(orow, col, kKPad / 8)) = o16.u;
      }
      report_range(go.status, vmax, kRangeResidual);
    }
    return;  // the hidden layer stays in LDS: nothing else reads it
  }
  const int kco = t.ldo >> 3;
  const int nch = (t_hi - t_lo) * 2;  // 8-column chunks of the group
  for (int uu = tid; uu < 16 * nch; uu += 512) {
    const int rr = uu / nch, ch = t_lo * 2 + uu % nch;
    if (m0 + rr < M)
      *reinterpret_cast<uint4*>(t.out16 + t16_off(m0 + rr, ch * 8, kco)) = *reinterpret_cast<const uint4*>(&sZ[rr][ch * 8]);
  }
}

hipError_t launch_step_boundary(const GemmArgs& v, const GemmArgs& t, const GemmArgs* o, hipStream_t s) {
  if (v.M < 1 || v.M != t.M || v.N != kAD || v.K < 1 || v.K > 8 * 3 * 32 || t.N != kD || t.K != kAD ||
      (v.wrs == nullptr) != (t.wrs == nullptr) || v.final_out || !v.x || !t.x || v.x == t.x ||
      (t.ow_rows > 0 && (!t.noise || !t.prev)))
    return hipErrorInvalidValue;
  if (o && (v.M > kBoundaryTimeOutMaxRows || o->M != v.M || o->N != kD || o->K != kD || !o->h || !o->h16 ||
            !o->bias || (o->wrs == nullptr) != (v.wrs == nullptr)))
    return hipErrorInvalidValue;
  BoundaryArgs ba;
  ba.v = v;
  ba.t = t;
  if (o) ba.o = *o;
  else memset(&ba.o, 0, sizeof(ba.o));
  const int nrb = (v.M + 15) / 16;
  if (o) {  // one workgroup per row block and 16-column block of the second layer
    const dim3 grid(nrb * (kD / 16)), block(512);
    if (v.wrs) hipLaunchKernelGGL((step_boundary_kernel<true, true>), grid, block, 0, s, ba);
    else hipLaunchKernelGGL((step_boundary_kernel<false, true>), grid, block, 0, s, ba);
    return hipGetLastError();
  }
  // column groups: up to 8 while the grid stays within one workgroup per CU
  const int G = nrb >= 128 ? 1 : (256 / nrb < 8 ? 256 / nrb : 8);
  const dim3 grid(nrb * G), block(512);
  if (v.wrs) hipLaunchKernelGGL((step_boundary_kernel<true>), grid, block, 0, s, ba);
  else hipLaunchKernelGGL((step_boundary_kernel<false>), grid, block, 0, s, ba);
  return hipGetLastError();
}

// FM = 16-row MFMA tiles per wave along M: BM = 32 * FM rows (two waves along M).
template <int AM, int EM, int FM>
__global__ __launch_bounds__(256, 2) void gemm_tiled(const GemmArgs a) {
  constexpr int BM = 32 * FM, BN = 128, BK = 64, LDC = BN + 4, CPR = BK / 8;
  constexpr int GA = BM * CPR / 256, GW = BN * CPR / 256;
  // LDS tiles keep the blocked layout: (r, c) at ((r / 16) * 8 + c / 8) * 128 + (r % 16) * 8 + c % 8,
  // so 16-byte piece g of a tile is at g * 8 both in LDS and (within a row block) in memory
  constexpr int STAGE = (BM + BN) * BK;  // halves
  constexpr int SMEM = 2 * STAGE * 2 > BM * LDC * 4 ? 2 * STAGE * 2 : BM * LDC * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
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

  uint4 ra[GA], rw[GW];
  float xmax = 0.f;  // A_X: the largest magnitude of the Euler state rounded to fp16
  // piece g of a tile: row (g / 128) * 16 + g % 16, chunk (g / 16) % 8
  auto prow = [](int g) { return ((g >> 7) << 4) | (g & 15); };
  auto pcol = [](int g) { return ((g >> 4) & (CPR - 1)) * 8; };
  auto load = [&](int kt) {
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < GA; ++i) {
      const int g = tid + 256 * i, row = m0 + prow(g), k = kb + pcol(g);
      const bool ok = row < M && k < K;
      ra[i] = load_a8<AM>(a, row, k, ok, 1.f, nt == 0, xmax);
    }
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = tid + 256 * i, n = n0 + prow(g), k = kb + pcol(g);
      rw[i] = (n < N && k < K) ? *reinterpret_cast<const uint4*>(a.W + t16_off(n, k, a.ldw >> 3)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    half_t* sA = stage0 + buf * STAGE;
    half_t* sW = sA + BM * BK;
#pragma unroll
    for (int i = 0; i < GA; ++i) {
      const int g = tid + 256 * i;
      *reinterpret_cast<uint4*>(sA + g * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = tid + 256 * i;
      *reinterpret_cast<uint4*>(sW + g * 8) = rw[i];
    }
  };

  f32x4 acc[FM][4];
  f32x4 sq[AM == A_NORM ? FM : 1];  // A_NORM: A A^T of each fm tile (row sums of squares on the diagonal)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if constexpr (AM == A_NORM) sq[fm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const half_t* sA = stage0 + (kt & 1) * STAGE;
    const half_t* sW = sA + BM * BK;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int ch = s * 4 + (lane >> 4);
      f16x8 af[FM], bw[4];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const f16x8*>(sA + ((wm * FM + fm) * CPR + ch) * 128 + (lane & 15) * 8);
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        bw[fn] = *reinterpret_cast<const f16x8*>(sW + ((wn * 4 + fn) * CPR + ch) * 128 + (lane & 15) * 8);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
      if constexpr (AM == A_NORM) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) sq[fm] = sumsq_mfma(af[fm], sq[fm]);
      }
    }
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  const float ws = a.w_scale;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wm * FM * 16 + fm * 16 + (lane >> 4) * 4 + r;
      float sc = ws;
      if constexpr (AM == A_NORM) sc *= rms_scale(a, diag_for_row(sq[fm], r, lane));
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) sC[rl * LDC + wn * 64 + fn * 16 + (lane & 15)] = acc[fm][fn][r] * sc;
    }
  __syncthreads();
  if constexpr (AM == A_X) report_range(a.status, xmax, kRangeTime);
  epilogue_tile<EM, BM, BN, LDC, 256>(a, sC, m0, n0);
}

GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p;
  const int nks = (K + 31) / 32;
  p.reg = 0;
  p.fmw = 2;
  p.bm = 64;
  p.rb = 4;
  p.cb = 1;
  p.stages = 2;
  if (M <= 64) {
    p.kind = 0;
    p.ntiles_n = (N + 15) / 16;
    const int need = (nks + 7) / 8;
    p.kpw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 6 ? 6 : need <= 8 ? 8
          : need <= 10 ? 10 : 0;
    // measured at 16 and 50 rows, with the operand just written by another kernel: one
    // 16-row block per workgroup is fastest for every projection (down 3.9 us against 5.8
    // with all rows in one workgroup, o 2.8 against 3.8, gate/up 4.2 against 4.6)
    p.rb = 1;
    // gate/up (N = 4096, weights from the last-level cache): two column blocks per workgroup
    // share the activation reads, 4.0 against 4.3 us (four: 4.1)
    p.cb = N >= 4096 ? 2 : 1;
  } else {
    p.kind = 1;
    p.ntiles_n = (N + 127) / 128;
    p.kpw = 0;
    p.bm = N <= 1024 ? 64 : 128;  // measured: 64-row tiles fill the chip better for N = 720/960
  }
  return p;
}

template <int AM, int EM, int RB, int CB, bool W8 = false>
static hipError_t launch_skinny(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  // E4M3 weights: the expert's projections only, at most two row and column blocks
  if constexpr (W8 && (RB > 2 || CB > 2 || EM == E_PF_QKV || EM == E_PF_RESID)) {
    (void)p; (void)a; (void)s;
    return hipErrorInvalidValue;
  } else {
  // column block groups rounded up to whole XCD rounds, times the row tiles (see gemm_skinny)
  const int groups = (p.ntiles_n + CB - 1) / CB, nrt = (a.M + 16 * RB - 1) / (16 * RB);
  const dim3 grid(8 * ((groups + 7) / 8) * nrt), block(512);
  switch (p.kpw) {
    case 1: hipLaunchKernelGGL((gemm_skinny<AM, EM, 1, RB, CB, W8>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_skinny<AM, EM, 2, RB, CB, W8>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_skinny<AM, EM, 3, RB, CB, W8>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_skinny<AM, EM, 4, RB, CB, W8>), grid, block, 0, s, a); break;
    case 6:
    case 8:
      // only the fp16-operand GEMMs have K > 1024 (down: K = 2048); the fp32-input
      // variants would not fit their fragments in registers
      // (64 x 64 tiles at K = 2048 would not fit their fragments in registers either)
      if constexpr (AM == A_F16 && RB * CB < 16) {
        if (p.kpw == 6) hipLaunchKernelGGL((gemm_skinny<AM, EM, 6, RB, CB, W8>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_skinny<AM, EM, 8, RB, CB, W8>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case 10:  // the prefix model's down projection (K = 2560), at most two 16 x 16 tiles per workgroup
      if constexpr (!W8 && AM == A_F16 && EM == E_PF_RESID && RB * CB <= 2) {
        hipLaunchKernelGGL((gemm_skinny<AM, EM, 10, RB, CB>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;  // K beyond 8 waves x 8 k-steps x 32
  }
  return hipGetLastError();
  }
}

template <int AM, int EM, int RB, bool W8>
static hipError_t launch_skinny_cb(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (p.cb) {
    case 1: return launch_skinny<AM, EM, RB, 1, W8>(p, a, s);
    case 2: return launch_skinny<AM, EM, RB, 2, W8>(p, a, s);
    case 4: return launch_skinny<AM, EM, RB, 4, W8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int AM, int EM, bool W8 = false>
static hipError_t launch_gemm_t(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  if (p.kind == 0) {
    switch (p.rb) {
      case 4: return launch_skinny_cb<AM, EM, 4, W8>(p, a, s);
      case 2: return launch_skinny_cb<AM, EM, 2, W8>(p, a, s);
      case 1: return launch_skinny_cb<AM, EM, 1, W8>(p, a, s);
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (W8) {
    return hipErrorInvalidValue;  // E4M3 weights: register-resident kernels only
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
  if (am == AMV && em == EMV) return a.wrs ? launch_gemm_t<AMV, EMV, true>(p, a, s) : launch_gemm_t<AMV, EMV>(p, a, s);
  SMOLEXP_GEMM_CASE(A_X, E_TIMEIN)
  SMOLEXP_GEMM_CASE(A_F16, E_H_BIAS)
  SMOLEXP_GEMM_CASE(A_NORM, E_QKV)
  SMOLEXP_GEMM_CASE(A_F16, E_H_RESID)
  SMOLEXP_GEMM_CASE(A_NORM, E_SWIGLU)
  SMOLEXP_GEMM_CASE(A_NORM, E_ACTOUT)
  SMOLEXP_GEMM_CASE(A_NORM, E_PF_QKV)
  SMOLEXP_GEMM_CASE(A_F16, E_PF_RESID)
#undef SMOLEXP_GEMM_CASE
  return hipErrorInvalidValue;
}


// Epilogue of a transposed accumulator tile (the weight fragment as the MFMA's first operand),
// for the residual projections: lane l of a wave holds, for each of its FMW x FN fragments, row
// r0 + 16 fm + l % 16 and the four consecutive columns c0 + 16 fn + 4 (l / 16) .. + 3, which is
// one 16-byte unit of the fp32 residual's 16 x 4 micro-tiles (and half of an 8-column chunk of
// its fp16 copy), so the sums go to memory from the registers (nontemporal stores) without
// staging the tile in LDS.  Measured against the staged epilogue, weights cycling through 256
// MB: o at 3200 rows 13.1 -> 12.4 us, down 23.5 -> 22.9, at 6400 rows 23.9 -> 22.5 and 38.0 ->
// 36.6; below 3200 rows and for the Q/K/V scatter (bf16 rows of 128 bytes, 27.6 against 18.4
// us) and the SwiGLU output (equal) the staged epilogue is kept.  rs: the scale of the lane's
// row in each row fragment.  PRE: the residual values were loaded before the main loop,
// pre[fm FN + fn].  Swapping the operands changes the rounding of a few fp32 sums (the
// matrix cores add the 32 products of a k-step in an order that depends on the operand
// roles), so the result equals the staged kernel's up to rounding, not bit for bit.
template <int FMW, int FN, bool PRE>
__device__ __forceinline__ void epilogue_regs_resid(const GemmArgs& a, const f32x4 (&acc)[FMW][FN],
                                                    const float (&rs)[FMW], int r0, int c0, int lane,
                                                    const float4* pre) {
  const int M = a.M, N = a.N;
  float vmax = 0.f;
#pragma unroll
  for (int fm = 0; fm < FMW; ++fm) {
    const int row = r0 + fm * 16 + (lane & 15);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = c0 + fn * 16 + 4 * (lane >> 4);
      if (row < M && col < N) {
        float4* hp = reinterpret_cast<float4*>(a.h + t32_off(row, col, kD / 4));
        const float4 hv = PRE ? pre[fm * FN + fn] : *hp;
        const float4 o = make_float4(hv.x + acc[fm][fn][0] * rs[fm], hv.y + acc[fm][fn][1] * rs[fm],
                                     hv.z + acc[fm][fn][2] * rs[fm], hv.w + acc[fm][fn][3] * rs[fm]);
        st_out<true>(hp, o);
        vmax = absmax4(vmax, o.x, o.y, o.z, o.w);
        union { half_t e[4]; uint2 u; } o16;
        o16.e[0] = (half_t)o.x; o16.e[1] = (half_t)o.y; o16.e[2] = (half_t)o.z; o16.e[3] = (half_t)o.w;
        st_out<true>(reinterpret_cast<uint2*>(a.h16 + t16_off(row, col, kKPad / 8)), o16.u);
      }
    }
  }
  report_range(a.status, vmax, kRangeResidual);
}

// ----------------------------------------------------------------------------
// Large-M GEMM with a multi-stage LDS pipeline
// ----------------------------------------------------------------------------
// BM x 128 tiles; each wave owns 16 FMW rows x 128 / WN columns.  The k-slabs
// (BK = 64 or 32 columns) rotate through an S-stage LDS ring filled by direct global->LDS
// loads (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at
// base + 16 l), so the next slabs are in flight while one is multiplied,
// without staging registers.  One load instruction moves four 16-row x
// 8-column micro-tiles (1 KB, contiguous in the blocked layout of both
// operands) and they land in LDS in the same blocked order, where the 16 lanes
// of a fragment read cover 256 consecutive bytes (no bank conflicts, no
// swizzle).  Requirements (checked by the launcher): A is fp16 with
// K % BK == 0 (K = 720 operands are zero-padded to 768).  With BK = 32 a stage holds half
// the columns, so the same LDS holds twice the stages: loads run further ahead of the
// matrix cores at the same occupancy, for one barrier per k-step instead of per two.  Waits are explicit:
// s_waitcnt vmcnt(n) + s_barrier, not __syncthreads (whose fence would wait
// for every load in flight).
constexpr int kBigBN = 128;
// Column groups of the tile -> XCD map (the rows are cut into 8 / GC groups).
__host__ __device__ constexpr int tile_col_groups(int em) { return em == E_SWIGLU ? 4 : 1; }

template <int EM, bool NORM, int BM, int FMW, int WN, int S, bool REG, int BK>
__global__ __launch_bounds__(64 * (BM / (16 * FMW)) * WN, 1) void gemm_big(const GemmArgs a) {
  constexpr int BN = kBigBN, LDC = BN + 4;
  constexpr int CH = BK / 8, LPR = CH / 4;  // 16-byte chunks per row of a slab; load instructions per row block
  static_assert(BK == 64 || BK == 32, "one or two k-steps per slab");
  constexpr int WM = BM / (16 * FMW), NW = WM * WN, FN = BN / 16 / WN;
  static_assert(WM * 16 * FMW == BM && FN * 16 * WN == BN, "waves tile the block");
  constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK * 2, STAGE_BYTES = A_BYTES + W_BYTES;
  // REG: the epilogue runs on the accumulators, the LDS holds only the ring
  constexpr int SMEM = REG || S * STAGE_BYTES > BM * LDC * 4 ? S * STAGE_BYTES : BM * LDC * 4;
  constexpr int A_LOADS = A_BYTES / 1024 / NW, W_LOADS = W_BYTES / 1024 / NW;  // per wave per stage
  constexpr int LOADS = A_LOADS + W_LOADS;
  static_assert(A_LOADS * NW * 1024 == A_BYTES && W_LOADS * NW * 1024 == W_BYTES, "whole load instructions per wave");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  float* sC = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w / WN, wn = w % WN;
  const int M = a.M, N = a.N, K = a.K;
  const int nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  // Tile -> XCD (workgroup i runs on XCD i % 8; j = i / 8 indexes that XCD's tiles).  GC = 1:
  // XCD x takes the x-th eighth of the tiles in row-major order.  GC > 1: the tile grid is
  // cut into 8 / GC row groups x GC column groups, one per XCD, each walked row by row;
  // gate/up (N = 4096) takes column quarters, so one XCD's L2 serves a 1.6 MB quarter of the
  // weights instead of streaming all 6.3 MB per row band.  Returns are uniform per
  // workgroup and come before any barrier.
  constexpr int GC = tile_col_groups(EM), GR = 8 / GC;
  const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  int mt, nt;
  if constexpr (GC == 1) {
    const int T = nM * nN, tile = xcd * ((T + 7) / 8) + j;
    if (tile >= T) return;
    mt = tile / nN;
    nt = tile % nN;
  } else {
    const int cg = xcd % GC, rg = xcd / GC;
    const int c_lo = cg * nN / GC, c_hi = (cg + 1) * nN / GC, r_lo = rg * nM / GR, r_hi = (rg + 1) * nM / GR;
    const int cw = c_hi - c_lo;
    if (cw <= 0 || j >= cw * (r_hi - r_lo)) return;
    mt = r_lo + j / cw;
    nt = c_lo + j % cw;
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk = K / BK;
  // E_H_RESID: the residual values this thread adds in the epilogue (its unit mapping: lane
  // r + 16 p of wave w owns row m0 + 16 w + r, columns n0 + 4 (p + 4 t)), loaded now so that
  // their latency hides behind the main loop.  Issued before the ring, they are the oldest
  // loads and the ring's vmcnt waits stay exact.  Only with the 4-stage ring, whose LDS
  // holds one workgroup per CU anyway: the 32 registers would halve the 2-stage ring's
  // occupancy (two workgroups per CU, 96 -> 132 VGPRs).
  constexpr bool PRE = (EM == E_H_RESID || EM == E_PF_RESID) && S > 2;
  float4 pre[PRE ? BN / 16 : 1];
  if constexpr (PRE && REG) {
    // REG mapping: lane l of wave (wm, wn) owns row m0 + (wm FMW + fm) 16 + l % 16 and columns
    // n0 + (wn FN + fn) 16 + 4 (l / 16) .. + 3 (pre[fm FN + fn])
    static_assert(FMW * FN <= BN / 16, "preloaded residual registers");
#pragma unroll
    for (int fm = 0; fm < FMW; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = m0 + (wm * FMW + fm) * 16 + (lane & 15), col = n0 + (wn * FN + fn) * 16 + 4 * (lane >> 4);
        if (row < M && col < N) pre[fm * FN + fn] = *reinterpret_cast<const float4*>(a.h + t32_off(row, col, resid_k4(EM)));
      }
  } else if constexpr (PRE) {
    static_assert(BM / 16 <= NW, "one row block per wave");
    const int row = m0 + w * 16 + (lane & 15);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      const int col = n0 + ((lane >> 4) + 4 * t) * 4;
      if (w < BM / 16 && row < M && col < N) pre[t] = *reinterpret_cast<const float4*>(a.h + t32_off(row, col, resid_k4(EM)));
    }
  }
  // NORM: A is fp16(h) unnormalised; each wave accumulates A A^T of its rows on the
  // matrix cores (row sums of squares on the diagonal), and 1/rms of each row scales the
  // finished sums.

  // Load instruction `blk` of a tile: row block blk / LPR, chunks (blk % LPR) * 4 .. +3 of the
  // slab; lane l moves row l % 16 of chunk l / 16 of those.  Row blocks past the last one holding
  // a row < M (or a column < N) are clamped to it: they only feed outputs that are not stored.
  const half_t* Ab = static_cast<const half_t*>(a.A);
  const int kcA = a.lda >> 3, kcW = a.ldw >> 3;
  const int rbA_last = (M - 1) >> 4, rbW_last = (N - 1) >> 4;
  auto issue = [&](int kt, int stage) {
    const int c0 = min(kt, nk - 1) * CH;  // past the end: reload the last slab (never read)
    char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int blk = w * A_LOADS + i;
      const int rb = min((m0 >> 4) + blk / LPR, rbA_last);
      const half_t* src = Ab + ((size_t)rb * kcA + c0 + (blk % LPR) * 4) * 128 + lane * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(base + blk * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i) {
      const int blk = w * W_LOADS + i;
      const int nb = min((n0 >> 4) + blk / LPR, rbW_last);
      const half_t* src = a.W + ((size_t)nb * kcW + c0 + (blk % LPR) * 4) * 128 + lane * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(base + A_BYTES + blk * 1024), 16, 0,
                                       0);
    }
  };

  f32x4 acc[FMW][FN];
  f32x4 sq[FMW];  // NORM: A A^T of each fm tile (row sums of squares on the diagonal)
#pragma unroll
  for (int fm = 0; fm < FMW; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = sq[fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of one 32-wide k-step, read from LDS into one of two register sets: the reads
  // of the next k-step are issued before the MFMAs of the current one (sched_barrier keeps
  // that order), so LDS latency hides behind 4 x FN MFMAs.
  auto read_frags = [&](int kt, int s, f16x8* af, f16x8* bw) {
    const char* base = smem + (kt % S) * STAGE_BYTES;
    const half_t* sA = reinterpret_cast<const half_t*>(base);
    const half_t* sW = reinterpret_cast<const half_t*>(base + A_BYTES);
    const int ch = s * 4 + (lane >> 4);  // 16-byte chunk of this lane's fragment within the slab
#pragma unroll
    for (int fm = 0; fm < FMW; ++fm)
      af[fm] = *reinterpret_cast<const f16x8*>(sA + ((wm * FMW + fm) * CH + ch) * 128 + (lane & 15) * 8);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      bw[fn] = *reinterpret_cast<const f16x8*>(sW + ((wn * FN + fn) * CH + ch) * 128 + (lane & 15) * 8);
  };
  // REG: the weight fragment is the MFMA's first operand, so the accumulator tile is C^T and
  // lane l holds row l % 16 with four consecutive columns 4 (l / 16) .. + 3
  // MFMAs lo .. hi - 1 of a k-step (fm-major over the FMW x FN tiles; the row sums of squares
  // with the last)
  auto mma_part = [&](const f16x8* af, const f16x8* bw, int lo, int hi) {
#pragma unroll
    for (int t = 0; t < FMW * FN; ++t) {
      if (t < lo || t >= hi) continue;
      const int fm = t / FN, fn = t % FN;
      if constexpr (REG) acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bw[fn], af[fm], acc[fm][fn], 0, 0, 0);
      else acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
    }
    if constexpr (NORM) {
      if (hi == FMW * FN) {
#pragma unroll
        for (int fm = 0; fm < FMW; ++fm) sq[fm] = sumsq_mfma(af[fm], sq[fm]);
      }
    }
  };
  auto mma = [&](const f16x8* af, const f16x8* bw) { mma_part(af, bw, 0, FMW * FN); };
  // Slabs kt + 1 .. kt + S - 1 are in flight while slab kt is multiplied; slab kt + S is
  // issued into slab kt's stage once every wave has finished reading it.  Past the end,
  // issue() reloads the last slab into a stage nobody reads any more, which keeps the counts
  // uniform.
  constexpr int WAIT1 = LOADS * (S - 2), WAIT2 = LOADS * (S - 1);
  static_assert(WAIT2 < 64, "vmcnt immediate range");
  constexpr int VM1 = (WAIT1 & 15) | ((WAIT1 >> 4) << 14), VM2 = (WAIT2 & 15) | ((WAIT2 >> 4) << 14);
#pragma unroll
  for (int st = 0; st < S; ++st) issue(st, st);
  __builtin_amdgcn_s_waitcnt(VM2 | (7 << 4) | (15 << 8));  // this wave's slab 0 landed
  __builtin_amdgcn_s_barrier();                            // ... every wave's
  f16x8 a0[FMW], b0[FN], a1[FMW], b1[FN];
  // The expert's RMSNorm'd operands hold 720 columns in K = 768: the second k-step of the
  // last slab (columns 736..767) is zero padding on both sides, and its MFMAs are skipped.
  const bool pad_tail = NORM && EM != E_PF_QKV && K == kKPad;
  read_frags(0, 0, a0, b0);
  if constexpr (BK == 64) {
    // In each half of a slab the first MFMA goes out before the next k-step's fragment reads:
    // the wait the compiler puts in front of it (always lgkmcnt(0) here: it counts the LDS-DMA
    // loads on that counter too) then covers only the fragments being multiplied.  Issued
    // before it, the reads were waited for as well, and every k-step waited for the next
    // one's reads before multiplying.  The last slab is peeled off so that the loop body has
    // no branch: at a branch's join the compiler assumes the worst path and waits again.
    for (int kt = 0; kt + 1 < nk; ++kt) {
      mma_part(a0, b0, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(kt, 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma_part(a0, b0, 1, FMW * FN);
      __builtin_amdgcn_sched_barrier(0);
      // this wave's reads of slab kt are done and its slab kt + 1 landed; then every wave's
      __builtin_amdgcn_s_waitcnt(VM1 | (7 << 4) | (0 << 8));
      __builtin_amdgcn_s_barrier();
      issue(kt + S, kt % S);
      __builtin_amdgcn_sched_barrier(0);
      mma_part(a1, b1, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(kt + 1, 0, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma_part(a1, b1, 1, FMW * FN);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma_part(a0, b0, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (!pad_tail) read_frags(nk - 1, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma_part(a0, b0, 1, FMW * FN);
    if (!pad_tail) mma(a1, b1);
  } else {
    // one k-step per slab: the same order (first MFMA, then the next slab's reads, then the
    // rest), with the barrier between the first MFMA and the reads
    const int nkc = pad_tail ? nk - 1 : nk;  // slabs multiplied
    auto step = [&](int kt, const f16x8* ca, const f16x8* cb, f16x8* na, f16x8* nb) {
      mma_part(ca, cb, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(VM1 | (7 << 4) | (0 << 8));
      __builtin_amdgcn_s_barrier();
      issue(kt + S, kt % S);
      read_frags(kt + 1, 0, na, nb);
      __builtin_amdgcn_sched_barrier(0);
      mma_part(ca, cb, 1, FMW * FN);
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 2 < nkc; kt += 2) {
      step(kt, a0, b0, a1, b1);
      step(kt + 1, a1, b1, a0, b0);
    }
    if (kt + 1 < nkc) {
      step(kt, a0, b0, a1, b1);
      mma(a1, b1);
    } else {
      mma(a0, b0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the trailing (unused) slabs must land before LDS is reused
  if constexpr (REG) {
    float rs[FMW];  // the weight scale (no RMSNorm on the residual projections)
#pragma unroll
    for (int fm = 0; fm < FMW; ++fm) rs[fm] = a.w_scale;
    static_assert(EM == E_H_RESID && !NORM, "register epilogue: the residual projections");
    epilogue_regs_resid<FMW, FN, PRE>(a, acc, rs, m0 + wm * FMW * 16, n0 + wn * FN * 16, lane, pre);
    return;
  }
  __syncthreads();

  const float ws = a.w_scale;
#pragma unroll
  for (int fm = 0; fm < FMW; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wm * 16 * FMW + fm * 16 + (lane >> 4) * 4 + r;
      float sc = ws;
      if constexpr (NORM) sc *= rms_scale(a, diag_for_row(sq[fm], r, lane));
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) sC[rl * LDC + (wn * FN + fn) * 16 + (lane & 15)] = acc[fm][fn][r] * sc;
    }
  __syncthreads();
  // nontemporal stores: the outputs of a round of tiles (megabytes) stream out instead of
  // sitting dirty in L2 until the end of the launch (batch 64 loop: 17.6 -> 16.4 ms; the
  // same stores in the small-batch kernels and the attention were slower or equal)
  epilogue_tile<EM, BM, BN, LDC, 64 * NW, PRE, true>(a, sC, m0, n0, pre);
}

template <int EM, bool NORM, int BM, int FMW, int WN, int S, bool REG = false, int BK = 64>
static hipError_t launch_gemm_dma(const GemmArgs& a, hipStream_t s) {
  constexpr int NT = 64 * (BM / (16 * FMW)) * WN, GC = tile_col_groups(EM), GR = 8 / GC;
  const int nM = (a.M + BM - 1) / BM, nN = (a.N + kBigBN - 1) / kBigBN;
  if (a.K % BK != 0 || a.lda % 8 != 0 || a.ldw % 8 != 0) return hipErrorInvalidValue;
  // every XCD gets as many workgroups as its largest share of tiles
  const int per = GC == 1 ? (nM * nN + 7) / 8 : ((nN + GC - 1) / GC) * ((nM + GR - 1) / GR);
  hipLaunchKernelGGL((gemm_big<EM, NORM, BM, FMW, WN, S, REG, BK>), dim3(8 * per), dim3(NT), 0, s, a);
  return hipGetLastError();
}

// Configurations: BM x 128 tiles of waves of 32 x 64 (eight waves at BM = 128, four at 64)
// and an S-stage ring.  Measured with the weights cycling through a 250 MB footprint,
// against 256-row tiles, four-wave 64 x 64 shapes and 3/4-stage rings: 128 rows and two
// 64-column stages (64 KB of LDS, two workgroups per CU) for Q/K/V and gate/up (gate/up at
// M = 3200: 29 us against 39 with a 4-stage ring); for o and down, whose 720 columns give few
// tiles, a 4-stage ring up to M = 4800 (down at 3200: 21.8 against 24.1 us) and 64-row tiles
// at M <= 2400 (down at 1600: 19.7 against 23.2).  Up to the denoising loop's 6400 rows the
// 128 x 128 Q/K/V and gate/up tiles hold four 32-column stages instead (the same 64 KB; three
// k-steps of loads ahead instead of two): batch 64 14.81 -> 14.66 ms, batch 128 23.57 ->
// 23.39, same bits; five stages were slower, and so was the prefix prefill's gate/up at 16448
// rows (7.665 -> 7.686 ms a call), which keeps the two 64-column stages.
constexpr int kSlab32MaxRows = 6400;
hipError_t launch_gemm_big(const GemmPlan& p, EMode em, bool norm, const GemmArgs& a, hipStream_t s) {
  const bool narrow = p.bm == 64 && p.fmw == 1;  // 64-row tiles of eight waves (16 rows each)
  switch (em) {
    case E_QKV:
      if (!norm) return hipErrorInvalidValue;
      if (narrow) return launch_gemm_dma<E_QKV, true, 64, 1, 2, 4>(a, s);
      if (a.M <= kSlab32MaxRows) return launch_gemm_dma<E_QKV, true, 128, 2, 2, 4, false, 32>(a, s);
      return launch_gemm_dma<E_QKV, true, 128, 2, 2, 2>(a, s);
    case E_SWIGLU:
      if (!norm) return hipErrorInvalidValue;
      if (narrow) return launch_gemm_dma<E_SWIGLU, true, 64, 1, 2, 4>(a, s);
      if (a.M <= kSlab32MaxRows) return launch_gemm_dma<E_SWIGLU, true, 128, 2, 2, 4, false, 32>(a, s);
      return launch_gemm_dma<E_SWIGLU, true, 128, 2, 2, 2>(a, s);
    case E_H_RESID:
      if (norm) return hipErrorInvalidValue;
      if (narrow) return launch_gemm_dma<E_H_RESID, false, 64, 1, 2, 4, true>(a, s);
      if (p.stages == 4) {
        if (p.reg) return launch_gemm_dma<E_H_RESID, false, 128, 2, 2, 4, true>(a, s);
        return launch_gemm_dma<E_H_RESID, false, 128, 2, 2, 4>(a, s);
      }
      if (p.reg) return launch_gemm_dma<E_H_RESID, false, 128, 2, 2, 2, true>(a, s);
      return launch_gemm_dma<E_H_RESID, false, 128, 2, 2, 2>(a, s);
    case E_PF_QKV:
      if (!norm) return hipErrorInvalidValue;
      return launch_gemm_dma<E_PF_QKV, true, 128, 2, 2, 2>(a, s);
    case E_PF_RESID:
      if (norm) return hipErrorInvalidValue;
      if (p.stages == 4) {
        if (p.bm == 64) return launch_gemm_dma<E_PF_RESID, false, 64, 2, 2, 4>(a, s);
        return launch_gemm_dma<E_PF_RESID, false, 128, 2, 2, 4>(a, s);
      }
      return launch_gemm_dma<E_PF_RESID, false, 128, 2, 2, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// The plan of one projection of the loop, from measurements with the weights cycling through a
// 256 MB footprint, as in the loop (us per launch, best kernel; the pipelined configurations are
// BM-row x 128-column tiles, eight waves, an S-stage ring):
//  * the register-resident K split (skinny) for the smallest row counts: Q/K/V 6.8 us at 400 rows
//    (8.0 pipelined), cross-layer Q 7.6 at 800 (8.1), o 7.9 at 1200 (8.7), down 13.1 at 800 (14.5);
//  * 64-row tiles of eight waves with a 4-stage ring (one workgroup per CU) wherever one round of
//    their tiles fits on the 256 CUs: Q/K/V at 800-1200 rows (8.4 / 9.4 against 11.9 / 15.9 for the
//    K split), cross-layer Q at 1200-2000 (8.6-9.2 against 10.4-16.2), gate/up at 400 (8.4 against
//    11.2), o at 1600-2400 (9.0-9.7 against 10.9-16.6 for the K split), down at 1200-2400
//    (15.1-17.6 against 17.9-20.2 for the 4-wave 64-row tiles);
//  * 128 x 128 tiles beyond: two stages (two workgroups per CU) for Q/K/V and gate/up; for o and
//    down, whose 720 columns give few tiles, four stages up to 4800 rows, with the epilogue from the
//    accumulators from 3200 rows on (down at 3200: 22.2 us);
//  * the register-staged tiled kernel only for the time MLP at 3200 rows and more.
// Row counts of whole rounds: 64-row tiles of a 720-column product fit one round up to 2688 rows
// (42 x 6 tiles), of the cross-layer Q (960 columns) up to 2048, of Q/K/V (1600) up to 1216, of
// gate/up (4096) up to 512.
GemmPlan plan_for(int M, int N, int K, AMode am, EMode em, bool w8) {
  GemmPlan p = plan_gemm(M <= 64 ? M : 64, N, K);  // skinny base: k-steps per wave, column blocks
  auto skinny = [&](int rb, int cb) {
    p.kind = 0; p.rb = rb; p.cb = cb;
    return p;
  };
  if (w8) {  // E4M3 weights (batches of at most 8 queries): the register-resident K split only
    // batch 1: the fp16 splits below (3.134 -> 3.095 ms a chunk)
    if (M <= 64) return em == E_SWIGLU ? skinny(2, 2) : em == E_QKV ? skinny(1, 2) : skinny(1, 1);
    return skinny(2, em == E_ACTOUT ? 1 : 2);
  }
  auto big = [&](int bm = 128, int stages = 2, int fmw = 2, int reg = 0) {
    GemmPlan b = p;
    b.kind = 2; b.bm = bm; b.stages = stages; b.fmw = fmw; b.reg = reg;
    return b;
  };
  // batch 1 (measured against one or two row blocks x one or two column blocks for each
  // projection, and 4 x 1, 1 x 4 for gate/up): gate/up on 32-row tiles of two column blocks
  // (4.38 -> 4.34 us a launch: half the workgroups reload the rows), Q/K/V on 16-row tiles of
  // two column blocks (3.34 -> 3.20 us); o, down and the time MLP keep one 16 x 16 block
  // (3.173 -> 3.153 ms a chunk)
  if (M <= 64) return em == E_SWIGLU ? skinny(2, 2) : em == E_QKV ? skinny(1, 2) : skinny(1, 1);
  (void)am;
  switch (em) {
    case E_QKV:
      if (N == kNQ) {  // cross layers: Q only
        if (M <= 1000) return skinny(2, 4);
        if (M <= 2048) return big(64, 4, 1);
      } else {
        if (M <= 600) return skinny(2, 2);
        if (M <= 1216) return big(64, 4, 1);
      }
      return big();
    case E_SWIGLU:
      if (M <= 300) return skinny(2, 2);
      return M <= 512 ? big(64, 4, 1) : big();
    case E_H_RESID:
      if (K > 1024) {  // down
        if (M <= 100) return skinny(2, 1);
        if (M <= 200) return skinny(2, 2);
        if (M <= 1000) return skinny(4, 2);
      } else {  // o
        if (M <= 400) return skinny(2, 2);
        if (M <= 1200) return skinny(4, 2);
      }
      if (M <= 2688) return big(64, 4, 1, 1);
      return M <= 4800 ? big(128, 4, 2, M >= 3200) : big(128, 2, 2, 1);
    case E_ACTOUT:
      if (M <= 2400) return skinny(1, 1);
      return M <= 4800 ? skinny(4, 2) : plan_gemm(M, N, K);
    default:  // time MLP
      return M <= 2400 ? skinny(2, 2) : plan_gemm(M, N, K);
  }
}

// ----------------------------------------------------------------------------
// Block-masked grouped-query attention
// ----------------------------------------------------------------------------
// The 150 query rows of KV head g are its 3 query heads x 50 chunk rows; a
// workgroup takes groups of 16 of them (one wave's tile) of one (query, KV
// head).  Keys are the prefix tokens 0..P-1 (valid where the mask says so)
// followed, in self layers, by the 50 chunk keys, of which row i sees j <= i.  Scores are computed
// transposed (S^T = K Q^T) so that each lane owns one query row; the output is
// accumulated transposed as well (O^T += V^T P^T).  K and V are staged in LDS
// row-major ([key][dim]); the V^T operand comes from transposing LDS reads.
constexpr int kKB = 64;        // keys per block
constexpr int kALD = kHD + 8;  // LDS row stride of K and V (elements)

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8-byte chunks addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and
// i / 4 + 12 of its group (checked on the device).  When lane s of a group
// addresses V[key0 + s / 4][d0 + 4 * (s % 4)], lane i therefore gets
// V[key0 .. key0 + 3][d0 + i]: four consecutive keys of one dimension.
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// One 64-key block of the online softmax for the lane's query row (row qi of
// the chunk).  sKb, sVb: the block's K and V rows [64][kALD]; kind: its key
// kinds; key0 = index of its first key minus P (chunk key j is visible to row
// qi when j - P <= qi).  MODE (uniform over the wave, from block_mode): 0 =
// every key is a valid prefix key (no mask), 1 = prefix keys only (valid or
// not), 2 = chunk keys too (causal test).  m_run: running max of the scaled
// scores (log2 domain); l_acc: running sum of the weights, accumulated on the
// matrix cores (an all-ones operand against the weights, so it sums exactly
// the bf16 weights that multiply V); every register holds it.
// Element (row, col) of a staged K or V block.  Padded layout: rows of kALD
// elements.  Swizzled layout (SWZ, filled by direct global->LDS loads that
// cannot pad): rows of 128 bytes whose 16-byte chunk c sits at c ^ (row % 8),
// so the 16 rows one fragment read touches spread over the banks.
template <bool SWZ>
__device__ __forceinline__ const bf16_t* kv_at(const bf16_t* base, int row, int col) {
  if constexpr (SWZ)
    return reinterpret_cast<const bf16_t*>(reinterpret_cast<const char*>(base) + row * 128 +
                                           ((((col >> 3) ^ row) & 7) << 4) + (col & 7) * 2);
  else
    return base + row * kALD + col;
}

template <int MODE, bool SWZ = false>
__device__ __forceinline__ void attn_block_m(const bf16_t* sKb, const bf16_t* sVb, const uint8_t* kind,
                                             int key0, int qi, const bf16x8* qf, f32x4* o, float& m_run,
                                             f32x4& l_acc, int lane) {
  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
  // S^T[key][row] for the 64 keys of the block (4 tiles of 16 keys)
  f32x4 sc[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    sc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = *reinterpret_cast<const uint4*>(kv_at<SWZ>(sKb, sub * 16 + (lane & 15), kk * 32 + (lane >> 4) * 8));
      sc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), qf[kk], sc[sub], 0, 0, 0);
    }
  }
  // masks (raw scores; the scale is positive, so the max commutes with it)
  if constexpr (MODE != 0) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int jl0 = sub * 16 + (lane >> 4) * 4;
      const unsigned k4 = *reinterpret_cast<const unsigned*>(kind + jl0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const unsigned kd = (k4 >> (8 * r)) & 0xffu;
        bool ok;
        if constexpr (MODE == 1) ok = kd == 1u;
        else ok = (kd == 1u) | ((kd == 2u) & ((key0 + jl0 + r) <= qi));
        sc[sub][r] = ok ? sc[sub][r] : -INFINITY;
      }
    }
  }
  float mb = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
  for (int sub = 1; sub < 4; ++sub) mb = fmaxf(fmaxf(mb, sc[sub][0]), fmaxf(fmaxf(sc[sub][1], sc[sub][2]), sc[sub][3]));
  mb = fmaxf(mb, __shfl_xor(mb, 16));
  mb = fmaxf(mb, __shfl_xor(mb, 32));
  const float m_new = fmaxf(m_run, mb * sl2);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  // v_exp_f32 directly: arguments are <= 0 and results that would be
  // denormal may flush to zero, which a softmax weight can afford
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
  for (int sub = 0; sub < 4; ++sub)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[sub][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[sub][r], sl2, -m_use));
  m_run = m_new;
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] *= alpha;
  l_acc[0] *= alpha;  // only register 0 is read back; the others are left to drift
  // O^T[d][row] += V^T[d][key] P^T[key][row], 32 keys per MFMA.  The k-slot
  // order (keys 4q..4q+3 then 16+4q..16+4q+3 for lane group q) is the same for
  // both operands.
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
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
      // V^T fragment: dims m*16 + (lane % 16), keys h2*32 + 4q .. +3 and +16 .. +19 (q = lane / 16)
      const int sl = lane & 15;
      const int vr = h2 * 32 + 4 * (lane >> 4) + (sl >> 2), vc = m * 16 + 4 * (sl & 3);
      const s16x4 lo = lds_read_tr16(kv_at<SWZ>(sVb, vr, vc)), hi = lds_read_tr16(kv_at<SWZ>(sVb, vr + 16, vc));
      const s16x4 u[2] = {lo, hi};
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), pb, o[m], 0, 0, 0);
    }
    l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, l_acc, 0, 0, 0);
  }
}

// How much masking a staged 64-key block needs (uniform over the wave): 0 when
// every key is a valid prefix key, 1 when all are prefix keys, 2 with chunk keys.
__device__ __forceinline__ int block_mode(const uint8_t* kind, int lane) {
  const unsigned k = kind[lane];
  if (__ballot(k == 2u) != 0ull) return 2;
  return __ballot(k != 1u) != 0ull ? 1 : 0;
}

template <bool SWZ = false>
__device__ __forceinline__ void attn_block(const bf16_t* sKb, const bf16_t* sVb, const uint8_t* kind,
                                           int key0, int qi, const bf16x8* qf, f32x4* o, float& m_run,
                                           f32x4& l_acc, int lane) {
  const int mode = block_mode(kind, lane);
  if (mode == 0) attn_block_m<0, SWZ>(sKb, sVb, kind, key0, qi, qf, o, m_run, l_acc, lane);
  else if (mode == 1) attn_block_m<1, SWZ>(sKb, sVb, kind, key0, qi, qf, o, m_run, l_acc, lane);
  else attn_block_m<2, SWZ>(sKb, sVb, kind, key0, qi, qf, o, m_run, l_acc, lane);
}

// Stage keys r0 .. r0 + RK - 1 of one (query, KV head) into LDS: K rows,
// V rows, key kinds.  Branch-free: every address is clamped into its
// buffer and the loaded vector is zeroed afterwards for masked or missing
// keys, so all loads are in flight together.  Split in two so that a caller
// can issue the loads early and store them to LDS later.
// The mask bytes are loaded unconditionally too (index clamped to P - 1; every call has P >= 1)
// and kept raw until store(): a byte load under a branch, compared at once, made the compiler
// wait for it, and so for every K/V load before it, one round trip per few vectors.
template <bool SELF, int RK, int NT>
struct AttnStage {
  static constexpr int NV = (RK * 8 + NT - 1) / NT;  // 16-byte vectors of K (and of V) per thread
  static constexpr int NKIND = (RK + NT - 1) / NT;
  uint4 kv[NV], vv[NV];
  unsigned mv[NV];     // mask byte of each vector's key (meaningful for prefix keys)
  unsigned mk[NKIND];  // mask byte of each kind entry's key
  int r0, P;

  __device__ __forceinline__ void issue(const AttnArgs& a, int b, int g, int r0_) {
    const int tid = threadIdx.x;
    r0 = r0_;
    P = a.P;
    const bf16_t* pk = a.pk + ((size_t)b * kHKV + g) * (size_t)P * kHD;
    const bf16_t* pv = a.pv + ((size_t)b * kHKV + g) * (size_t)P * kHD;
    const bf16_t* ck = SELF ? a.kc + ((size_t)b * kHKV + g) * kChunk * kHD : pk;
    const bf16_t* cv = SELF ? a.vc + ((size_t)b * kHKV + g) * kChunk * kHD : pv;
    const uint8_t* m = a.mask + (size_t)b * P;
#pragma unroll
    for (int it = 0; it < NKIND; ++it) {
      const int j = r0 + tid + NT * it;
      mk[it] = m[j < P ? j : P - 1];
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int v = min(tid + NT * it, RK * 8 - 1);  // past the end: repeat the last vector (not stored)
      // K and V rows: 8 lanes per key (whole 128-byte rows)
      const int j = r0 + (v >> 3), c = (v & 7) * 8;
      const bool pre = j < P, chunk = SELF && !pre && j - P < kChunk;
      // 32-bit element offsets from the head's base pointers (P <= 4096 keys of 64 elements):
      // cheaper address arithmetic ahead of the loads than 64-bit offsets
      const unsigned po = pre ? (unsigned)(j * kHD + c) : (unsigned)c, co = (unsigned)((j - P) * kHD + c);
      kv[it] = *reinterpret_cast<const uint4*>(chunk ? ck + co : pk + po);
      vv[it] = *reinterpret_cast<const uint4*>(chunk ? cv + co : pv + po);
      mv[it] = m[pre ? j : P - 1];
    }
  }
  __device__ __forceinline__ void store(bf16_t* sK, bf16_t* sV, uint8_t* sKind) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < NKIND; ++it) {
      const int j = r0 + tid + NT * it;
      const uint8_t kind = j < P ? (mk[it] ? 1 : 0) : ((SELF && j - P < kChunk) ? 2 : 0);
      if (tid + NT * it < RK) sKind[tid + NT * it] = kind;
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int v = tid + NT * it;
      const int j = r0 + (min(v, RK * 8 - 1) >> 3);
      const bool pre = j < P, chunk = SELF && !pre && j - P < kChunk;
      const bool kok = pre ? mv[it] != 0 : chunk;
      if (!kok) kv[it] = vv[it] = make_uint4(0, 0, 0, 0);
      if (NV * NT == RK * 8 || v < RK * 8) {
        *reinterpret_cast<uint4*>(sK + (v >> 3) * kALD + (v & 7) * 8) = kv[it];
        *reinterpret_cast<uint4*>(sV + (v >> 3) * kALD + (v & 7) * 8) = vv[it];
      }
    }
  }
};

template <bool SELF, int RK, int NT = 256>
__device__ __forceinline__ void attn_stage(const AttnArgs& a, int b, int g, int r0, bf16_t* sK, bf16_t* sV,
                                           uint8_t* sKind) {
  AttnStage<SELF, RK, NT> st;
  st.issue(a, b, g, r0);
  st.store(sK, sV, sKind);
}

// Small batches: a workgroup takes QG groups of 16 query rows of one KV head
// (of its 3 x 50) and KS waves per group split the staged key blocks among
// themselves (wave (q, k) takes blocks k, k + KS, ...); with KS > 1 each
// group's softmax states (running max, running sum, unnormalised output) are
// merged through LDS.  All QG x KS waves share one staging of the keys.
template <bool SELF, int NBLK, int QG, int KS>
__global__ __launch_bounds__(64 * QG * KS) void attn_small_kernel(const AttnArgs a) {
  constexpr int NT = 64 * QG * KS, RK = NBLK * kKB, OLD = kHD + 4;
  constexpr int KV_BYTES = 2 * RK * kALD * 2, MERGE_BYTES = KS > 1 ? QG * KS * 16 * OLD * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[KV_BYTES > MERGE_BYTES ? KV_BYTES : MERGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[RK];
  __shared__ float sM[QG][KS][16], sL[QG][KS][16];
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem);  // K rows, then V rows
  bf16_t* sV = sK + RK * kALD;
  float* sO = reinterpret_cast<float*>(smem);    // [QG][KS][16][OLD], used after the last round

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qg = wave / KS, ks = wave % KS;
  // one-dimensional grid: the RG row groups of one (query, KV head) unit get the same
  // i % 8 (workgroup i runs on XCD i % 8), so the K/V they all stage come through one L2;
  // the return is uniform per workgroup and comes before any barrier
  constexpr int RG = (3 * kChunk + 16 * QG - 1) / (16 * QG);
  const int xcd = (int)(blockIdx.x & 7), jx = (int)(blockIdx.x >> 3);
  const int u = 8 * (jx / RG) + xcd, rgx = jx % RG;
  if (u >= kHKV * a.B) return;
  const int g = u % kHKV, b = u / kHKV;
  const int P = a.P;
  // the first round's key loads go out first: the setup below (the loop's invariants
  // included) runs while they are in flight
  AttnStage<SELF, RK, NT> st;
  st.issue(a, b, g, 0);
  __builtin_amdgcn_sched_barrier(0);
  const int rq = rgx * (16 * QG) + qg * 16 + (lane & 15);
  const bool rvalid = rq < 3 * kChunk;
  const int hq = 3 * g + (rvalid ? rq / kChunk : 0);
  const int qi = rvalid ? rq % kChunk : 0;

  bf16x8 qf[2];
  {
    // loaded for every lane (a row past the end reads row 0 of the group's first head) and
    // zeroed after, with no branch around the loads
    const bf16_t* qp = a.q + (((size_t)b * kHQ + hq) * kChunk + qi) * kHD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = *reinterpret_cast<const uint4*>(qp + kk * 32);
      qf[kk] = __builtin_bit_cast(bf16x8, rvalid ? u : make_uint4(0, 0, 0, 0));
    }
  }
  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  f32x4 l_acc = f32x4{0.f, 0.f, 0.f, 0.f};

  const int NK = P + (SELF ? kChunk : 0);
  for (int r0 = 0; r0 < NK; r0 += RK) {
    // before a later round, every wave must be done with the previous round's keys (the first
    // round's loads were issued above, with nothing in LDS to protect)
    if (r0 > 0) {
      __syncthreads();
      st.issue(a, b, g, r0);
    }
    st.store(sK, sV, sKind);
    __syncthreads();
    const int nb = min(NBLK, (NK - r0 + kKB - 1) / kKB);
    for (int blk = ks; blk < nb; blk += KS)
      attn_block(sK + blk * kKB * kALD, sV + blk * kKB * kALD, sKind + blk * kKB, r0 + blk * kKB - P, qi, qf, o,
                 m_run, l_acc, lane);
  }

  float vmax = 0.f;
  if constexpr (KS == 1) {
    if (rvalid) {
      const float l_run = l_acc[0];
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      const int orow = b * kChunk + qi;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
        for (int r = 0; r < 4; ++r) pk4.h[r] = (half_t)(o[m][r] * inv);
        vmax = absmax4(vmax, o[m][0] * inv, o[m][1] * inv, o[m][2] * inv, o[m][3] * inv);
        *reinterpret_cast<uint2*>(a.out + t16_off(orow, hq * kHD + m * 16 + (lane >> 4) * 4, kNQ / 8)) = pk4.u;
      }
    }
  } else {
    // merge the KS waves' states of each query group
    __syncthreads();
    if (lane < 16) {
      sM[qg][ks][lane] = m_run;
      sL[qg][ks][lane] = l_acc[0];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sO[((qg * KS + ks) * 16 + (lane & 15)) * OLD + m * 16 + (lane >> 4) * 4 + r] = o[m][r];
    __syncthreads();
    for (int u = tid; u < QG * 16 * 16; u += NT) {
      const int q2 = u >> 8, row = (u >> 4) & 15, d0 = (u & 15) * 4;
      const int rq2 = rgx * (16 * QG) + q2 * 16 + row;
      if (rq2 >= 3 * kChunk) continue;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < KS; ++w) mx = fmaxf(mx, sM[q2][w][row]);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        const float sc = __builtin_amdgcn_exp2f(sM[q2][w][row] - mu);
        l += sL[q2][w][row] * sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += sO[((q2 * KS + w) * 16 + row) * OLD + d0 + e] * sc;
      }
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int hq2 = 3 * g + rq2 / kChunk, qi2 = rq2 % kChunk;
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk4.h[e] = (half_t)(acc[e] * inv);
      vmax = absmax4(vmax, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<uint2*>(a.out + t16_off(b * kChunk + qi2, hq2 * kHD + d0, kNQ / 8)) = pk4.u;
    }
  }
  report_range(a.status, vmax, kRangeAttention);
}

template <bool SELF, int QG, int KS>
static void launch_small(const AttnArgs& a, hipStream_t s) {
  // key blocks staged per round: the whole key range when it fits in five blocks
  const int nk = a.P + (SELF ? kChunk : 0);
  const int nblk = min(5, max(2, (nk + kKB - 1) / kKB));
  const int RG = (3 * kChunk + 16 * QG - 1) / (16 * QG);
  const dim3 grid(8 * RG * ((kHKV * a.B + 7) / 8)), block(64 * QG * KS);
  switch (nblk) {
    case 2: hipLaunchKernelGGL((attn_small_kernel<SELF, 2, QG, KS>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((attn_small_kernel<SELF, 3, QG, KS>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_small_kernel<SELF, 4, QG, KS>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attn_small_kernel<SELF, 5, QG, KS>), grid, block, 0, s, a); break;
  }
}

// Measured at batch 1 (graph replay, P = 177): four key-split waves per query group beat
// fewer, wider workgroups; self layers gain a little from two query groups per workgroup
// (4.9 against 5.1 us), cross layers do not.
template <bool SELF>
static void launch_ksplit(const AttnArgs& a, hipStream_t s) {
  if constexpr (SELF) launch_small<SELF, 2, 4>(a, s);
  else launch_small<SELF, 1, 4>(a, s);
}

// Cross-attention layer of a small batch with its own query projection: the
// keys of a cross layer come only from the prefix cache, so the Q/K/V GEMM of
// that layer (which computes only Q there) needs no other workgroup's results
// and one launch does both.  A workgroup takes 16 rows of one query head:
//  (1) it issues the loads of its projection operands (16 rows of fp16(h),
//      the head's 64 weight rows, 8 waves splitting K = 768 as the M <= 64
//      GEMM does) together with the first round of prefix K/V;
//  (2) the projection runs on the matrix cores, the row sums of squares from
//      A A^T; the waves' partials meet in LDS, where the 1/rms scale and the
//      rotary embedding are applied and Q is rounded to bf16;
//  (3) the 8 waves split the staged key blocks (online softmax as above) and
//      merge their states in LDS.
// The Q values equal those of the separate GEMM launch (same K split, same
// order of the sums).
// W8: the Q weights are E4M3 codes with row scales (as gemm_skinny's W8).
template <int NBLK, bool W8 = false>
__global__ __launch_bounds__(512) void attn_cross_q_kernel(const AttnArgs a) {
  constexpr int NT = 512, NW = 8, RK = NBLK * kKB, OLD = kHD + 4, QLD = kHD + 8;
  constexpr int KPW = kKPad / 32 / NW;  // k-steps per wave
  static_assert(KPW * 32 * NW == kKPad, "K split");
  constexpr int KV_BYTES = 2 * RK * kALD * 2;
  constexpr int RED_BYTES = NW * 16 * kHD * 4, MERGE_BYTES = NW * 16 * OLD * 4;
  __shared__ __attribute__((aligned(16))) char sKV[KV_BYTES];
  __shared__ __attribute__((aligned(16))) char sR[RED_BYTES > MERGE_BYTES ? RED_BYTES : MERGE_BYTES];
  __shared__ __attribute__((aligned(16))) bf16_t sQt[16 * QLD];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[RK];
  __shared__ float sQ[NW][16], sM[NW][16], sL[NW][16];
  bf16_t* sK = reinterpret_cast<bf16_t*>(sKV);
  bf16_t* sV = sK + RK * kALD;
  float* sRed = reinterpret_cast<float*>(sR);  // [wave][row][64] projection partials
  float* sO = reinterpret_cast<float*>(sR);    // [wave][row][OLD] after the last round

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // one-dimensional grid: the 3 heads x RB row blocks of one (query, KV head) unit get the
  // same i % 8 (workgroup i runs on XCD i % 8): each head's weight slice and the unit's K/V
  // come through one L2; the return is uniform per workgroup and comes before any barrier
  constexpr int RB = (kChunk + 15) / 16;
  const int xcd = (int)(blockIdx.x & 7), jx = (int)(blockIdx.x >> 3);
  const int u = 8 * (jx / (3 * RB)) + xcd, rr = jx % (3 * RB);
  if (u >= kHKV * a.B) return;
  const int g = u % kHKV, b = u / kHKV, hq = 3 * g + rr / RB, rb = rr % RB;
  const int P = a.P;

  // the weight scales of the two output columns this thread finishes in (2)
  float ws1 = a.w_scale, ws2 = a.w_scale;
  if constexpr (W8) {
    const int c1 = ((tid & 31) >> 3) * 16 + (tid & 7);
    ws1 = a.wrs[hq * kHD + c1];
    ws2 = a.wrs[hq * kHD + c1 + 8];
  }
  // (1) projection operands of this wave's K slice, then the first round of keys
  const int qa = rb * 16 + (lane & 15);  // chunk row of this lane's A fragment
  const bool aok = qa < kChunk;
  uint4 af[KPW];
  WFrag<W8> wf[KPW][4];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int k = (w * KPW + i) * 32 + (lane >> 4) * 8;
    // every lane loads (rows past the chunk read the query's row 0) and the value is zeroed
    // after, with no branch around the load
    const uint4 av = *reinterpret_cast<const uint4*>(a.h16 + t16_off(b * kChunk + (aok ? qa : 0), k, kKPad / 8));
    af[i] = aok ? av : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      wf[i][cb] = load_wfrag<W8>(a.wq, t16_off(hq * kHD + cb * 16 + (lane & 15), k, a.ldw >> 3), true);
  }
  AttnStage<false, RK, NT> st;
  st.issue(a, b, g, 0);
  // the key loads go out before the projection's MFMAs, whose operand waits would otherwise
  // hold them back until the projection operands had arrived
  __builtin_amdgcn_sched_barrier(0);

  // (2) Q = fp16(h) W'^T on the matrix cores, and the rows' sums of squares
  f32x4 acc[4], sq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const f16x8 av = __builtin_bit_cast(f16x8, af[i]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, w_to_f16x8(wf[i][cb])), acc[cb], 0, 0, 0);
    sq = sumsq_mfma(av, sq);
  }
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sRed[(w * 16 + (lane >> 4) * 4 + r) * kHD + cb * 16 + (lane & 15)] = acc[cb][r];
  if (((lane & 15) >> 2) == (lane >> 4)) sQ[w][lane & 15] = sq[lane & 3];
  st.store(sK, sV, sKind);
  __syncthreads();
  {
    // thread -> (row, rotation pair d): weight rows of block d / 8 hold dims d0..d0+7 then d0+32..
    const int r = tid >> 5, d = tid & 31, qr = rb * 16 + r;
    const int c1 = (d >> 3) * 16 + (d & 7), c2 = c1 + 8;
    float s1 = 0.f, s2 = 0.f, q = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      s1 += sRed[(w2 * 16 + r) * kHD + c1];
      s2 += sRed[(w2 * 16 + r) * kHD + c2];
      q += sQ[w2][r];
    }
    bf16_t lo = 0, hi = 0;
    if (qr < kChunk) {
      const float rs = rms_scale_qk(a.inv_k, a.eps, q);
      const float v1 = s1 * (ws1 * rs), v2 = s2 * (ws2 * rs);
      const float2 cs = a.ropeq[(size_t)(b * kChunk + qr) * (kHD / 2) + d];
      lo = f2bf(v1 * cs.x - v2 * cs.y);
      hi = f2bf(v1 * cs.y + v2 * cs.x);
    }
    sQt[r * QLD + d] = lo;
    sQt[r * QLD + d + kHD / 2] = hi;
  }
  __syncthreads();

  // (3) attention of the 16 rows over the prefix keys
  const int qi = rb * 16 + (lane & 15);
  bf16x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sQt + (lane & 15) * QLD + kk * 32 + (lane >> 4) * 8));
  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  f32x4 l_acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < P; r0 += RK) {
    if (r0 > 0) {
      __syncthreads();
      attn_stage<false, RK, NT>(a, b, g, r0, sK, sV, sKind);
      __syncthreads();
    }
    const int nb = min(NBLK, (P - r0 + kKB - 1) / kKB);
    for (int blk = w; blk < nb; blk += NW)
      attn_block(sK + blk * kKB * kALD, sV + blk * kKB * kALD, sKind + blk * kKB, r0 + blk * kKB - P, qi, qf, o,
                 m_run, l_acc, lane);
  }
  __syncthreads();
  if (lane < 16) {
    sM[w][lane] = m_run;
    sL[w][lane] = l_acc[0];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(w * 16 + (lane & 15)) * OLD + m * 16 + (lane >> 4) * 4 + r] = o[m][r];
  __syncthreads();
  if (tid < 16 * 16) {
    const int row = tid >> 4, d0 = (tid & 15) * 4, qr = rb * 16 + row;
    if (qr < kChunk) {
      float mx = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) mx = fmaxf(mx, sM[w2][row]);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float l = 0.f, acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float sc = __builtin_amdgcn_exp2f(sM[w2][row] - mu);
        l += sL[w2][row] * sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc4[e] += sO[(w2 * 16 + row) * OLD + d0 + e] * sc;
      }
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk4.h[e] = (half_t)(acc4[e] * inv);
      *reinterpret_cast<uint2*>(a.out + t16_off(b * kChunk + qr, hq * kHD + d0, kNQ / 8)) = pk4.u;
      report_range(a.status, absmax4(0.f, acc4[0] * inv, acc4[1] * inv, acc4[2] * inv, acc4[3] * inv),
                   kRangeAttention);
    }
  }
}

// Batches above 8: one workgroup per (16 NW query rows, KV head g, query b);
// its NW waves take 16 rows each (the 150 rows of KV head g are its 3 query
// heads x 50 chunk rows; NW = 10 takes them all).  The 64-key blocks stream through an S-stage LDS ring by
// direct global->LDS loads (swizzled rows, kv_at<true>): while block j is
// multiplied, the loads of blocks j+1 .. j+S-1 are in flight, so a block costs
// about one barrier instead of one memory round trip (staging one block per
// round through registers, as the small-batch kernels do, cost half the time of
// a batch-64 launch: 19 us with it, 10 with the staging loads switched off).  The kinds of all keys
// are staged once.  A block holding keys that are not attended (masked prefix
// keys, or the clamped keys past the end) has their V rows zeroed in LDS before
// use: their weights are 0, but 0 x NaN would not be.
constexpr int kMaxKeys = 4096 + 64;  // max_prefix + the chunk, in whole blocks

template <bool SELF, int S, int MINB = 1, int NW = 4, bool PF = false>
__global__ __launch_bounds__(64 * NW, MINB) void attn_pipe_kernel(const AttnArgs a) {
  static_assert(!(PF && SELF), "a prefill's keys are the prefix alone");
  constexpr int NT = 64 * NW, BLK_BYTES = kKB * kHD * 2, STAGE = 2 * BLK_BYTES;
  constexpr int NLOAD = STAGE / 1024;              // 1 KB load instructions per stage
  constexpr int LPW = (NLOAD + NW - 1) / NW;      // per wave (the last waves may issue fewer)
  static_assert(S >= 2, "ring depth");
  constexpr int WAITN = (S - 2) * LPW;    // this wave's loads still allowed in flight
  constexpr int VMW = (WAITN & 15) | ((WAITN >> 4) << 14);
  __shared__ __attribute__((aligned(1024))) char ring[S * STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[kMaxKeys];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // One-dimensional grid: workgroup i runs on XCD i % 8, and the RG row groups of one
  // (query, KV head) unit u get the same i % 8, so they stage the same K/V blocks through
  // one L2 (fetched from memory once, not once per row group).  The return is uniform per
  // workgroup and comes before any barrier.  The query rows of a KV head are its 3 query
  // heads x seq rows: the chunk's 50, or (PF) the P prefix tokens of a prefill.
  const int seq = PF ? a.seq : kChunk;
  const int RG = PF ? (3 * seq + 16 * NW - 1) / (16 * NW) : (3 * kChunk + 16 * NW - 1) / (16 * NW);
  const int xcd = (int)(blockIdx.x & 7), jx = (int)(blockIdx.x >> 3);
  const int u = 8 * (jx / RG) + xcd, rgi = jx % RG;
  if (u >= kHKV * a.B) return;
  const int g = u % kHKV, b = u / kHKV, P = a.P;
  const int NK = P + (SELF ? kChunk : 0), nblk = (NK + kKB - 1) / kKB;
  const int rq = rgi * (16 * NW) + w * 16 + (lane & 15);
  const bool rvalid = rq < 3 * seq;
  const int hq = 3 * g + (rvalid ? rq / seq : 0);
  const int qi = rvalid ? rq % seq : 0;

  // key kinds: 0 = none, 1 = valid prefix key, 2 = chunk key
  const uint8_t* mk = a.mask + (size_t)b * P;
  for (int j = tid; j < nblk * kKB; j += NT)
    sKind[j] = j < P ? (mk[j] ? 1 : 0) : ((SELF && j - P < kChunk) ? 2 : 0);

  // element offsets from pk: the V rows of the prefix, the chunk's K rows and their V rows
  const size_t head = (size_t)b * kHKV + g;
  const bf16_t* pk = a.pk + head * (size_t)P * kHD;
  const ptrdiff_t pv_off = (a.pv + head * (size_t)P * kHD) - pk;
  const ptrdiff_t ck_off = SELF ? (a.kc + head * kChunk * kHD) - pk : 0;
  const ptrdiff_t cv_off = SELF ? (a.vc + head * kChunk * kHD) - pk : 0;
  // Load instruction i of a stage (wave w issues i = w LPW .. w LPW + LPW - 1): part i / 8
  // (K, then V), LDS rows 8 (i % 8) .. +7; lane l fills LDS row 8 (i % 8) + l / 8, chunk
  // l % 8, i.e. global chunk (l % 8) ^ (row % 8) of that key.  Keys past the last are
  // clamped to it (kind 0).  Blocks past the last reload the last one (never read).
  auto issue = [&](int blk, int stage) {
    const int bb = min(blk, nblk - 1);
    char* base = ring + stage * STAGE;
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int i = w * LPW + t, part = i >> 3;
      if (NLOAD % NW != 0 && i >= NLOAD) break;  // uniform per wave
      const int row = (i & 7) * 8 + (lane >> 3), chunk = (lane & 7) ^ (row & 7);
      const int key = min(bb * kKB + row, NK - 1);
      const bool pre = !SELF || key < P;
      const ptrdiff_t off = (pre ? (part ? pv_off : 0) + (ptrdiff_t)key * kHD
                                 : (part ? cv_off : ck_off) + (ptrdiff_t)(key - P) * kHD) + chunk * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(pk + off),
                                       (__attribute__((address_space(3))) void*)(base + part * BLK_BYTES + (i & 7) * 1024),
                                       16, 0, 0);
    }
  };

  bf16x8 qf[2];
  {
    const bf16_t* qp = a.q + (((size_t)b * kHQ + hq) * seq + qi) * kHD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 u = rvalid ? *reinterpret_cast<const uint4*>(qp + kk * 32) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  f32x4 l_acc = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st);
  for (int j = 0; j < nblk; ++j) {
    __builtin_amdgcn_s_waitcnt(VMW | (7 << 4) | (0 << 8));  // this wave's loads of block j (and LDS writes) done
    __builtin_amdgcn_s_barrier();                           // everyone's; block j - 1 finished everywhere
    const uint8_t* kb = sKind + j * kKB;
    const bf16_t* sK = reinterpret_cast<const bf16_t*>(ring + (j % S) * STAGE);
    const bf16_t* sV = sK + BLK_BYTES / 2;
    if (__ballot(kb[lane] == 0u) != 0ull) {  // uniform: some keys of this block are not attended
      for (int u = tid; u < kKB * 8; u += NT)
        if (kb[u >> 3] == 0u)
          *reinterpret_cast<uint4*>(ring + (j % S) * STAGE + BLK_BYTES + (u >> 3) * 128 + (u & 7) * 16) = make_uint4(0, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(VMW | (7 << 4) | (0 << 8));
      __builtin_amdgcn_s_barrier();
    }
    issue(j + S - 1, (j + S - 1) % S);  // into the stage block j - 1 used
    attn_block<true>(sK, sV, kb, j * kKB - P, qi, qf, o, m_run, l_acc, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the trailing (unused) loads land before the LDS is released

  if (rvalid) {
    const float l_run = l_acc[0];
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    const int orow = b * seq + qi;
    float vmax = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int r = 0; r < 4; ++r) pk4.h[r] = (half_t)(o[m][r] * inv);
      vmax = absmax4(vmax, o[m][0] * inv, o[m][1] * inv, o[m][2] * inv, o[m][3] * inv);
      *reinterpret_cast<uint2*>(a.out + t16_off(orow, hq * kHD + m * 16 + (lane >> 4) * 4, kNQ / 8)) = pk4.u;
    }
    report_range(a.status, vmax, kRangeAttention);
  }
}

// The same streamed attention with the K/V blocks staged through registers into two LDS
// stages: while block j is multiplied, block j + 1 is already in LDS and block j + 2 is in
// flight in registers, stored to LDS after block j (keys that are not attended zeroed on the
// way).  With direct global->LDS loads in flight the compiler
// makes the block's LDS reads (the transposing V^T reads among them) wait for every load, so the
// next block's loads never overlapped the current block's arithmetic; register loads carry no
// such wait.  Same scores, same sums, same bits as attn_pipe_kernel.
// One 64-key block of K and V staged through registers: vector i of a thread is v = tid + NT i
// (v < 512), key row v / 8, 16-byte chunk v % 8.  issue(): every load unconditional, keys past
// the last clamped to it; store(): into an LDS stage in the swizzled layout of kv_at<true>
// (chunk c of row r at c ^ (r % 8)), keys whose kind (the LDS key-kind table) is 0 zeroed.
template <bool SELF, int NT>
struct StreamStage {
  static constexpr int NVEC = kKB * kHD / 8, NV = (NVEC + NT - 1) / NT;
  uint4 k[NV], v[NV];
  __device__ __forceinline__ void issue(const bf16_t* pk, const bf16_t* pv, const bf16_t* ck, const bf16_t* cv,
                                        int P, int NK, int bb) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vv = min(tid + NT * i, NVEC - 1);
      const int key = min(bb * kKB + (vv >> 3), NK - 1), c = (vv & 7) * 8;
      const bool pre = !SELF || key < P;
      const unsigned po = (unsigned)(key * kHD + c), co = (unsigned)((key - P) * kHD + c);
      k[i] = *reinterpret_cast<const uint4*>(pre ? pk + po : ck + co);
      v[i] = *reinterpret_cast<const uint4*>(pre ? pv + po : cv + co);
    }
  }
  __device__ __forceinline__ void store(char* base, int blk_bytes, const uint8_t* kind) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vv = tid + NT * i;
      const int row = (vv >> 3) & (kKB - 1);
      const bool ok = kind[row] != 0;
      const int off = row * 128 + ((((vv & 7) ^ row) & 7) << 4);
      // component-wise selects: a select of whole uint4 values became a select of their
      // addresses and kept the staging registers in scratch memory
      const unsigned keep = ok ? ~0u : 0u;
      if (NVEC % NT == 0 || vv < NVEC) {
        *reinterpret_cast<uint4*>(base + off) = make_uint4(k[i].x & keep, k[i].y & keep, k[i].z & keep, k[i].w & keep);
        *reinterpret_cast<uint4*>(base + blk_bytes + off) =
            make_uint4(v[i].x & keep, v[i].y & keep, v[i].z & keep, v[i].w & keep);
      }
    }
  }
};

// The same streamed attention with the K/V blocks staged through registers into two LDS
// stages: while block j is multiplied from one stage, block j + 1 is in flight in registers and
// is stored into the other stage after block j (keys that are not attended zeroed on the way,
// from the key-kind table), then block j + 2's loads are issued.  With direct global->LDS loads in flight the compiler
// makes the block's LDS reads (the transposing V^T reads among them) wait for every load, so the
// next block's loads never overlapped the current block's arithmetic; register loads carry no
// such wait.  Same scores, same sums, same bits as attn_pipe_kernel.
template <bool SELF, int MINB = 1, int NW = 4, bool PF = false>
__global__ __launch_bounds__(64 * NW, MINB) void attn_stream_kernel(const AttnArgs a) {
  static_assert(!(PF && SELF), "a prefill's keys are the prefix alone");
  constexpr int NT = 64 * NW, BLK_BYTES = kKB * kHD * 2, STAGE = 2 * BLK_BYTES;
  constexpr int RW = 16 * NW;                   // query rows per workgroup
  __shared__ __attribute__((aligned(1024))) char ring[2 * STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sKind[kMaxKeys];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // grid: as attn_pipe_kernel (the RG row groups of a (query, KV head) unit on one XCD)
  const int seq = PF ? a.seq : kChunk;
  const int RG = (3 * seq + RW - 1) / RW;
  const int xcd = (int)(blockIdx.x & 7), jx = (int)(blockIdx.x >> 3);
  const int u = 8 * (jx / RG) + xcd, rgi = jx % RG;
  if (u >= kHKV * a.B) return;
  const int g = u % kHKV, b = u / kHKV, P = a.P;
  const int NK = P + (SELF ? kChunk : 0), nblk = (NK + kKB - 1) / kKB;
  const int rq = rgi * RW + w * 16 + (lane & 15);
  const bool rvalid = rq < 3 * seq;
  const int hq = 3 * g + (rvalid ? rq / seq : 0);
  const int qi = rvalid ? rq % seq : 0;

  const uint8_t* mk = a.mask + (size_t)b * P;
  const size_t head = (size_t)b * kHKV + g;
  const bf16_t* pk = a.pk + head * (size_t)P * kHD;
  const bf16_t* pv = a.pv + head * (size_t)P * kHD;
  const bf16_t* ck = SELF ? a.kc + head * kChunk * kHD : pk;
  const bf16_t* cv = SELF ? a.vc + head * kChunk * kHD : pv;
  StreamStage<SELF, NT> st;

  // The first block's keys and the Q rows go out together (a row past the last reads query row 0
  // of head 3 g: its results are never stored); the key-kind fill waits for them (its mask loads
  // are conditional), then the first block goes into LDS and the second block's loads are issued,
  // in flight through the first block's arithmetic.
  st.issue(pk, pv, ck, cv, P, NK, 0);
  bf16x8 qf[2];
  {
    const bf16_t* qp = a.q + (((size_t)b * kHQ + hq) * seq + qi) * kHD + (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + kk * 32));
  }
  __builtin_amdgcn_sched_barrier(0);
  // key kinds: 0 = none, 1 = valid prefix key, 2 = chunk key
  for (int j = tid; j < nblk * kKB; j += NT)
    sKind[j] = j < P ? (mk[j] ? 1 : 0) : ((SELF && j - P < kChunk) ? 2 : 0);
  __syncthreads();  // the kinds, for every thread's stores
  // every load so far has landed (the first block's store needs them anyway): the loop then
  // never waits for the Q fragments behind the next block's loads
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  st.store(ring, BLK_BYTES, sKind);
  if (nblk > 1) st.issue(pk, pv, ck, cv, P, NK, 1);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  f32x4 l_acc = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < nblk; ++j) {
    __syncthreads();  // block j stored by every thread; block j - 1 finished by every wave
    const bf16_t* sK = reinterpret_cast<const bf16_t*>(ring + (j & 1) * STAGE);
    attn_block<true>(sK, sK + BLK_BYTES / 2, sKind + j * kKB, j * kKB - P, qi, qf, o, m_run, l_acc, lane);
    if (j + 1 < nblk) {  // uniform
      st.store(ring + ((j + 1) & 1) * STAGE, BLK_BYTES, sKind + (j + 1) * kKB);  // the stage block j - 1 used
      if (j + 2 < nblk) st.issue(pk, pv, ck, cv, P, NK, j + 2);
    }
  }

  if (rvalid) {
    const float l_run = l_acc[0];
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    const int orow = b * seq + qi;
    float vmax = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      union { half_t h[4]; uint2 u; } pk4;
#pragma unroll
      for (int r = 0; r < 4; ++r) pk4.h[r] = (half_t)(o[m][r] * inv);
      vmax = absmax4(vmax, o[m][0] * inv, o[m][1] * inv, o[m][2] * inv, o[m][3] * inv);
      *reinterpret_cast<uint2*>(a.out + t16_off(orow, hq * kHD + m * 16 + (lane >> 4) * 4, kNQ / 8)) = pk4.u;
    }
    report_range(a.status, vmax, kRangeAttention);
  }
}

// Grid of attn_pipe_kernel: 8 XCD lanes x RG row groups x ceil(5 B / 8) units.
static dim3 pipe_grid(int B, int NW, int seq = kChunk) {
  const int RG = (3 * seq + 16 * NW - 1) / (16 * NW);
  return dim3(8 * RG * ((kHKV * B + 7) / 8));
}

// Variants by batch, from a sweep at P = 177 and 257 with the one-dimensional
// XCD-grouped grid (us per launch, self / cross at P = 177): four waves and a 3-stage
// ring up to batch 16 (7.2 / 5.2); five waves, two workgroups per CU at 24 (7.4 / 5.8
// against 8.6 / 6.6 with ten); ten waves (each block loaded once for all 150 rows of a
// KV head) at 33-48 and 65-96 rows of queries, where 5 B such workgroups fill the CUs
// in whole rounds (batch 48: 9.1 / 7.0 against 10.9 / 7.8); otherwise four waves with
// registers capped for four workgroups per CU (batch 64: 13.2 / 9.7 against 16.5 /
// 12.3 with ten; batch 128: 23.5 / 17.5 against 25.2 / 19.4).  Before the grid kept
// the row groups of a (query, KV head) on one XCD, batch 64 took 20.0 / 19.1 us at
// P = 257 in the loop against 15.8 / 14.5 now.  The register-staged kernel (attn_stream_kernel)
// replaces the ring where its registers still allow the same workgroups per CU: up to batch 24
// (batch 16, variable prefixes <= 241, whole call 8.48 -> 8.21 ms; batch 24 9.80 -> 9.60) and
// with ten waves (batch 40 10.89 -> 10.75); with four waves and four workgroups per CU it would
// spill, and at three per CU batch 32 (two per call at batch 64) measured equal and batch 64 (at
// batch 128) slower (15.5 / 11.6 -> 15.8 / 12.4 us per launch, two rounds of workgroups).
template <bool SELF>
static void launch_pipe(const AttnArgs& a, hipStream_t s) {
  const int B = a.B;
  if (B <= 16) hipLaunchKernelGGL((attn_stream_kernel<SELF, 1, 4>), pipe_grid(B, 4), dim3(256), 0, s, a);
  else if (B <= 24) hipLaunchKernelGGL((attn_stream_kernel<SELF, 2, 5>), pipe_grid(B, 5), dim3(320), 0, s, a);
  else if ((B > 32 && B <= 48) || (B > 64 && B <= 96))
    hipLaunchKernelGGL((attn_stream_kernel<SELF, 1, 10>), pipe_grid(B, 10), dim3(640), 0, s, a);
  else hipLaunchKernelGGL((attn_pipe_kernel<SELF, 2, 4>), pipe_grid(B, 4), dim3(256), 0, s, a);
}

// A prefill's prefix self-attention: 3 P query rows per KV head, four-wave workgroups of
// 64 rows, keys = the valid prefix tokens in both directions (the prefix is one block of the
// block mask).
hipError_t launch_prefix_attention(const AttnArgs& a, hipStream_t s) {
  if (a.B < 1 || a.P < 1 || a.seq != a.P || a.P + kKB > kMaxKeys) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_pipe_kernel<false, 2, 4, 4, true>), pipe_grid(a.B, 4, a.seq), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool W8>
static void launch_cross_q_t(const AttnArgs& a, hipStream_t s) {
  const int nblk = min(5, max(2, (a.P + kKB - 1) / kKB));
  const int RB = (kChunk + 15) / 16;
  const dim3 grid(8 * 3 * RB * ((kHKV * a.B + 7) / 8)), block(512);
  switch (nblk) {
    case 2: hipLaunchKernelGGL((attn_cross_q_kernel<2, W8>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((attn_cross_q_kernel<3, W8>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_cross_q_kernel<4, W8>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attn_cross_q_kernel<5, W8>), grid, block, 0, s, a); break;
  }
}

static void launch_cross_q(const AttnArgs& a, hipStream_t s) {
  if (a.wrs) launch_cross_q_t<true>(a, s);
  else launch_cross_q_t<false>(a, s);
}

bool use_cross_q(int B) { return B <= kCrossQMaxBatch; }

hipError_t launch_attention(bool self_layer, const AttnArgs& a, hipStream_t s) {
  if (!self_layer && a.wq) {  // cross layer with its query projection
    if (!use_cross_q(a.B) || !a.h16 || !a.ropeq || a.ldw != kKPad) return hipErrorInvalidValue;
    launch_cross_q(a, s);
    return hipGetLastError();
  }
  if (a.B <= 8) {
    if (self_layer) launch_ksplit<true>(a, s);
    else launch_ksplit<false>(a, s);
  } else {
    if (self_layer) launch_pipe<true>(a, s);
    else launch_pipe<false>(a, s);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Prologue: the time vectors W_t1[:, 720:] e(t_k) + b_t1 for n_t flow times
// (the schedule's once, when the weights are loaded; one per velocity call),
// and per call the RoPE rows of every chunk row (position = the query's number
// of valid prefix tokens + i) and x <- the caller's x.
// ----------------------------------------------------------------------------
constexpr int kTimeRowsPerBlock = 16;
constexpr int kTimeBlocks = kD / kTimeRowsPerBlock;  // 45

__global__ __launch_bounds__(256) void prologue_kernel(const PrologueArgs a) {
  __shared__ float se[kD];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = 0;  // every later kernel of the call follows this one
  const int nMaskBlocks = (a.B + 3) / 4;
  const int timeBlocks = a.n_t > 0 ? kTimeBlocks : 0;
  if ((int)blockIdx.x < timeBlocks) {
    // Sinusoidal time embedding: sin(2 pi t / p_i) for i < 360, cos(...) after,
    // periods geometric from p_min to p_max (1/p_i precomputed in fp64).  The
    // angle is reduced to [0, 2 pi) in fp64, then sin/cos run in fp32.
    // Row j of W_t1[:, 720:] is read once, 8 halves per lane, for every step.
    const int j = blockIdx.x * kTimeRowsPerBlock + (tid >> 4), part = tid & 15;
    const half_t* wr = a.w_t1e + (size_t)j * kD;
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
  } else if ((int)blockIdx.x < timeBlocks + nMaskBlocks) {
    // query b: its valid prefix count n, then the RoPE rows of chunk positions n .. n + 49
    // Loads are issued in batches before their values are used: a loop that loads and then
    // stores (or accumulates) each element in turn waits for every load on its own, since the
    // compiler cannot move a load above a store that may alias it.
    const int b = (blockIdx.x - timeBlocks) * 4 + (tid >> 6), lane = tid & 63;
    if (b < a.B) {
      const uint8_t* mrow = a.mask + (size_t)b * a.P;
      constexpr int MU = 4;  // mask bytes per lane and batch: P <= 256 in one
      int c = 0;
      for (int j0 = 0; j0 < a.P; j0 += 64 * MU) {
        unsigned mb[MU];
#pragma unroll
        for (int u = 0; u < MU; ++u) {
          const int j = j0 + lane + 64 * u;
          mb[u] = mrow[j < a.P ? j : a.P - 1];
        }
#pragma unroll
        for (int u = 0; u < MU; ++u) c += (j0 + lane + 64 * u < a.P) && mb[u] != 0u;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
      constexpr int RU = kChunk * (kHD / 2) / 64;  // RoPE entries per lane
      static_assert(RU * 64 == kChunk * (kHD / 2), "whole rows per lane");
      float2 rv[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) rv[u] = a.rope[(size_t)c * (kHD / 2) + lane + 64 * u];
#pragma unroll
      for (int u = 0; u < RU; ++u) a.ropeq[((size_t)b * kChunk) * (kHD / 2) + lane + 64 * u] = rv[u];
    }
  } else {
    const int first = timeBlocks + nMaskBlocks;
    const int n = a.B * kChunk * kAD;
    for (int i = (blockIdx.x - first) * 256 + tid; i < n; i += (gridDim.x - first) * 256) a.x[i] = a.x_in[i];
  }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  const int nMaskBlocks = (a.B + 3) / 4;
  const int nCopy = (a.B * kChunk * kAD + 255) / 256;
  const int copyBlocks = nCopy < 64 ? nCopy : 64;
  const int blocks = (a.n_t > 0 ? kTimeBlocks : 0) + nMaskBlocks + copyBlocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prologue_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Prefill of the prefix language model
// ----------------------------------------------------------------------------
// Prologue, positions: workgroup (x, b) takes prefix tokens j0 = 64 x .. j0 + 63 of query b
// and writes each token's RoPE row at its position (the number of valid tokens before it in
// the query: a count of the mask before j0, then a running sum over the 64).
__global__ __launch_bounds__(256) void prefill_rope_rows_kernel(const PrefillPrologueArgs a) {
  const int b = blockIdx.y, j0 = blockIdx.x * 64, tid = threadIdx.x, P = a.P;
  if (b == 0 && blockIdx.x == 0 && tid == 0 && a.status) *a.status = 0;  // the prefill's first kernel
  const uint8_t* mk = a.mask + (size_t)b * P;
  __shared__ int sCnt[256];
  __shared__ int sPos[64];
  int c = 0;
  for (int j = tid; j < j0; j += 256) c += mk[j] ? 1 : 0;
  sCnt[tid] = c;
  if (tid < 64) sPos[tid] = (j0 + tid < P && mk[j0 + tid]) ? 1 : 0;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sCnt[tid] += sCnt[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    int run = sCnt[0];
    for (int i = 0; i < 64; ++i) {
      const int f = sPos[i];
      sPos[i] = run;
      run += f;
    }
  }
  __syncthreads();
  for (int e = tid; e < 64 * (kHD / 2); e += 256) {
    const int i = e / (kHD / 2), d = e % (kHD / 2), j = j0 + i;
    if (j < P) a.ropeq[((size_t)b * P + j) * (kHD / 2) + d] = a.rope[(size_t)sPos[i] * (kHD / 2) + d];
  }
}

// Prologue, residual: each thread converts 4 consecutive columns of one token's bf16
// embedding to the fp32 residual and its fp16 copy (blocked, 960 columns); 16 consecutive
// lanes take 16 consecutive rows of one column chunk, as the blocked layouts store them.
__global__ __launch_bounds__(256) void prefill_embed_kernel(const PrefillPrologueArgs a) {
  const size_t rows = (size_t)a.B * a.P, units = ((rows + 15) / 16) * 16 * (kLmD / 4);
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (size_t)gridDim.x * 256) {
    const size_t blk = u / (16 * (kLmD / 4)), rem = u % (16 * (kLmD / 4));
    const int c4 = (int)(rem / 16);
    const size_t row = blk * 16 + rem % 16;
    if (row >= rows) continue;
    const uint2 raw = *reinterpret_cast<const uint2*>(a.emb + row * kLmD + c4 * 4);
    const float4 v = make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                                 __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u));
    *reinterpret_cast<float4*>(a.h + t32_off((int)row, c4 * 4, kLmD / 4)) = v;
    report_range(a.status, absmax4(0.f, v.x, v.y, v.z, v.w), kRangeResidual);
    union { half_t e[4]; uint2 u; } o16;
    o16.e[0] = (half_t)v.x; o16.e[1] = (half_t)v.y; o16.e[2] = (half_t)v.z; o16.e[3] = (half_t)v.w;
    *reinterpret_cast<uint2*>(a.h16 + t16_off((int)row, c4 * 4, kLmD / 8)) = o16.u;
  }
}

hipError_t launch_prefill_prologue(const PrefillPrologueArgs& a, hipStream_t s) {
  if (a.B < 1 || a.P < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_rope_rows_kernel, dim3((a.P + 63) / 64, a.B), dim3(256), 0, s, a);
  const size_t units = (((size_t)a.B * a.P + 15) / 16) * 16 * (kLmD / 4);
  const size_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(prefill_embed_kernel, dim3(blocks < 4096 ? (unsigned)blocks : 4096u), dim3(256), 0, s, a);
  return hipGetLastError();
}

// The prefill's projections, M = B P rows, from a sweep at 177-2832 rows (us per launch,
// weights rotating; skinny rb x cb against the pipelined kernel): Q/K/V skinny 2 x 2 up to 600
// rows (177: 5.7), pipelined above (708: 12.8, 2832: 18.4, where 2 x 2 takes 47); o 2 x 2 up
// to 400, 4 x 2 up to 1000 (708: 6.8), then 64-row and 128-row 4-stage tiles (1416: 10.1,
// 2832: 13.1); gate/up 2 x 4 up to 300 rows (177: 7.7 against 12.0 pipelined), pipelined
// above (1416: 18.2 against 34.0); down (K = 2560, ten k-steps per wave, at most two tiles
// per workgroup) 1 x 2 up to 800 rows (708: 19.9), then 64-row and 128-row 4-stage tiles;
// beyond 4800 rows o and down take the 2-stage ring as in the expert (two workgroups per CU).
GemmPlan plan_prefill(int M, int N, int K, EMode em) {
  GemmPlan p = plan_gemm(M <= 64 ? M : 64, N, K);
  auto skinny = [&](int rb, int cb) {
    p.kind = 0; p.rb = rb; p.cb = cb;
    return p;
  };
  auto big = [&](int bm, int stages) {
    GemmPlan b = p;
    b.kind = 2; b.bm = bm; b.stages = stages;
    return b;
  };
  if (M <= 64) return skinny(1, em == E_SWIGLU ? 2 : 1);
  switch (em) {
    case E_PF_QKV:
      return M <= 600 ? skinny(2, 2) : big(128, 2);
    case E_SWIGLU:
      return M <= 300 ? skinny(2, 4) : big(128, 2);
    case E_PF_RESID:
      if (K > kLmD) {  // down
        if (M <= 800) return skinny(1, 2);
      } else {  // o
        if (M <= 400) return skinny(2, 2);
        if (M <= 1000) return skinny(4, 2);
      }
      return M <= 2400 ? big(64, 4) : M <= 4800 ? big(128, 4) : big(128, 2);  // many tiles: two workgroups per CU
    default:
      return big(128, 2);
  }
}

// ----------------------------------------------------------------------------
// Workspace of the no-alloc denoise: a fixed array of device memory, one copy on every GPU
// the library runs on, held until the process ends.  In host code `scratch` only names the
// symbol: its device address is looked up once per device, with that device current, and
// kept; kernels receive that address.
// ----------------------------------------------------------------------------
constexpr size_t kNoAllocBytes = call_ws_bytes(kNoAllocMaxBatch);
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(int device, char** ptr, size_t* bytes) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = static_cast<char*>(p);
  }
  *ptr = g_scratch_ptr[device];
  *bytes = kNoAllocBytes;
  return hipSuccess;
}

// Columns 720..767 of h16 are chunks 90..95 of each 16-row block: 6 x 256 contiguous bytes.
__global__ __launch_bounds__(256) void zero_h16_pad_kernel(half_t* h16, int nblk) {
  constexpr int kPieces = (kKPad - kD) / 8 * 16;  // 16-byte pieces per row block
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk * kPieces) return;
  const int rb = i / kPieces, j = i % kPieces;
  reinterpret_cast<uint4*>(h16 + ((size_t)rb * (kKPad / 8) + kD / 8) * 128)[j] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_h16_pad(half_t* h16, int rows, hipStream_t s) {
  if (rows <= 0 || rows % 16 != 0) return hipErrorInvalidValue;
  const int n = rows / 16 * ((kKPad - kD) / 8 * 16);
  hipLaunchKernelGGL(zero_h16_pad_kernel, dim3((n + 255) / 256), dim3(256), 0, s, h16, rows / 16);
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
