// tmx_rankmixer.hip -- the RankMixer block on gfx950 (fun-rec chapter 7.4.0
// block equations; 7.4.1 token mixing with H = T as the reproduction guide's
// section 5 requires; 7.4.2 per-token FFN with biases; 7.4.3 ReLU routing):
//
//   S      = rho(LN_1(TokenMixing(X) + X))
//   X_next = rho(LN_2(S + rho(GELU(S W1_t + b1_t)) W2_t + b2_t))
//
// or, with E ReLU-routed experts per token (inference router),
//   X_next = rho(LN_2(S + sum_j [rho(G_j GELU(S W1_tj + b1_tj)) W2_tj + G_j b2_tj])),
//   G = ReLU(S Wr_t).
//
// One kernel per block. A workgroup owns 64 samples of one token t:
//  * prologue: each wave forms 16 rows of TokenMixing(X) + X straight from X
//    (the mixing map folded into the loads), LayerNorm in fp32, S rounded to
//    bf16 into LDS -- S is both the FFN input and its residual; with experts
//    the router logits and gates follow;
//  * per hidden chunk of 128: GEMM1 (W1 fragments as the MFMA A operand, S
//    rows as B, so each lane's accumulators hold 4 consecutive hidden units
//    of one row), bias + GELU (erf by a published rational approximation,
//    below) [x gate], the rounded chunk into LDS; GEMM2 the same way round
//    (W2 fragments as A, the hidden chunk as B) accumulating the token's
//    whole output row set in registers;
//  * epilogue: bias + residual S, LayerNorm statistics reduced across lanes
//    and waves in fixed order, rounding, the tile staged through LDS and
//    written with 16-byte row-contiguous stores.
// Tile order is XCD-aware: consecutive workgroups of one XCD share a token,
// so its 2 * D * kD weights stay in that XCD's L2.
#include "tmx_internal.h"

namespace tmx {
namespace {

constexpr int RMX_BM = 64;    // samples per workgroup
// waves per workgroup and hidden units per chunk: 4 and 128 at D = 256 (two
// workgroups per CU), 8 and 256 at D = 512 (one workgroup per CU, still two
// waves per SIMD, each wave on a 64-column eighth); every wave owns 32 hidden
// units of a chunk and 64 output columns
constexpr int rmx_waves(int D) { return D / 64; }
constexpr int rmx_chunk(int D) { return 32 * rmx_waves(D); }
constexpr int RMX_HC = 128;   // chunk of the expert path (D = 256)

template <int D, int EM = 0>
struct RmxShape {
  static constexpr int EPL = D / 64;           // row elements per lane in a row pass
  static constexpr int SA = D + 8;             // LDS row stride of S (bf16 elements)
  static constexpr int NW = rmx_waves(D);      // waves per workgroup
  static constexpr int HC = rmx_chunk(D);      // hidden units per chunk
  static constexpr int SU = HC + 8;            // LDS row stride of a hidden chunk
  static constexpr int KT1 = D / 16;           // GEMM1 K steps (over D)
  static constexpr int NT2 = D / 32 / NW;      // GEMM2 output column tiles per wave
  static constexpr int KT2 = HC / 16;          // GEMM2 K steps per chunk
  static constexpr int BYTES_S = RMX_BM * SA * 2;
  static constexpr int BYTES_U = RMX_BM * SU * 2;
  static constexpr int BYTES_RED = 2 * NW * RMX_BM * 4;
  // ReLU-routed experts (EM experts per token): each row's gates as bf16
  // hi | lo pairs (g = hi + lo to 16 significant bits), [64][2 EM + 8], and
  // one "any row active" flag per expert
  static constexpr int SG = 2 * EM + 8;
  static constexpr int BYTES_G = EM ? RMX_BM * SG * 2 + EM * 4 : 0;
  static constexpr int LDS = BYTES_S + 2 * BYTES_U + BYTES_RED + BYTES_G;
};

template <int N> struct VecOf;
template <> struct VecOf<4> { typedef uint2 type; };
template <> struct VecOf<8> { typedef uint4 type; };

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// GELU z * Phi(z) in fp32, Phi(z) = (1 + erf(z / sqrt 2)) / 2, with erf from
// Abramowitz & Stegun formula 7.1.26 (Hastings' rational approximation):
// for x >= 0, erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x), |error| <= 1.5e-7. Written for the lower tail,
// q = erfc(|z| / sqrt 2) / 2 = Phi(-|z|), so Phi(z) = z < 0 ? q : 1 - q keeps
// full relative accuracy for negative z. One reciprocal and one exp2 per
// value against about three times the instructions of the library erff.
__device__ __forceinline__ float gelu_erf(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  // coefficients a1..a5 halved (the 1/2 of q folded in)
  float p = fmaf(t, 0.5307027145f, -0.7265760135f);
  p = fmaf(t, p, 0.7107068705f);
  p = fmaf(t, p, -0.1422483680f);
  p = fmaf(t, p, 0.1274147960f);
  const float q = p * t * __builtin_amdgcn_exp2f(-x * x * 1.4426950408889634f);
  return z * (z < 0.f ? q : 1.0f - q);
}

template <int EPL>
__device__ __forceinline__ void unpack_row(const typename VecOf<EPL>::type& q, float* v) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&q);
#pragma unroll
  for (int i = 0; i < EPL / 2; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// S row of token t, sample b, columns [EPL * lane, +EPL): LayerNorm of
// TokenMixing(X) + X (fp32 statistics over the wave), rounded to bf16.
// TokenMixing with H = T: column c = t' * dh + j of mixed token t is
// X[b, t', t * dh + j]; EPL consecutive columns stay inside one dh segment.
template <int D>
__device__ __forceinline__ typename VecOf<D / 64>::type ln1_row(const typename VecOf<D / 64>::type& xq,
                                                                const typename VecOf<D / 64>::type& mq,
                                                                const float* g, const float* be, float eps) {
  constexpr int EPL = D / 64;
  float a[EPL], m[EPL];
  unpack_row<EPL>(xq, a);
  unpack_row<EPL>(mq, m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    a[i] += m[i];
    s += a[i];
  }
  const float mean = wsum(s) * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    a[i] -= mean;
    q += a[i] * a[i];
  }
  const float rstd = 1.0f / sqrtf(wsum(q) * (1.0f / D) + eps);
  typename VecOf<EPL>::type o;
  uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
  for (int i = 0; i < EPL / 2; ++i)
    ow[i] = pack_bf16x2(a[2 * i] * rstd * g[2 * i] + be[2 * i], a[2 * i + 1] * rstd * g[2 * i + 1] + be[2 * i + 1]);
  return o;
}

// the mixed row t of sample b is position t of the Mix map (H = T)
template <int D>
__device__ __forceinline__ int64_t mix_offset(int64_t b, int t, int T, int dh, int c0) {
  return RowMap{T, D, dh, 1}.offset(b, t, c0);
}

// ---------------------------------------------------------------------------
// sub-layer 0 alone: S = rho(LN_1(TokenMixing(X) + X)); one wave per row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rmx_ln1_kernel(RmxArgs a) {
  constexpr int EPL = D / 64;
  typedef typename VecOf<EPL>::type Vec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.T) return;
  const int64_t b = row / a.T;
  const int t = (int)(row - b * a.T);
  const int c0 = lane * EPL;
  float g[EPL], be[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    g[i] = a.g1[c0 + i];
    be[i] = a.be1[c0 + i];
  }
  const Vec xq = *reinterpret_cast<const Vec*>(a.x + row * D + c0);
  const Vec mq = *reinterpret_cast<const Vec*>(a.x + mix_offset<D>(b, t, a.T, a.dh, c0));
  *reinterpret_cast<Vec*>(a.out + row * D + c0) = ln1_row<D>(xq, mq, g, be, a.eps);
}

// ---------------------------------------------------------------------------
// the block (FUSED: from X) or its FFN sub-layer (from S); EM > 0: the FFN is
// EM ReLU-routed experts of hidden a.h_e per token (D = 256 only)
// ---------------------------------------------------------------------------
template <int D, bool FUSED, int EM, bool ROUTE = false>
__global__ __launch_bounds__(64 * rmx_waves(D), D <= 256 ? 2 : 1) void rmx_block_kernel(RmxArgs a) {
  static_assert(EM == 0 || D == 256, "the expert path is laid out for D = 256");
  typedef RmxShape<D, EM> S_;
  constexpr int EPL = S_::EPL, SA = S_::SA, SU = S_::SU, KT1 = S_::KT1, NT2 = S_::NT2, KT2 = S_::KT2;
  constexpr int NW = S_::NW, HC = S_::HC, RPW = RMX_BM / NW;   // RPW: prologue rows per wave
  static_assert(EM == 0 || HC == RMX_HC, "the expert path runs 128-unit chunks");
  typedef typename VecOf<EPL>::type Vec;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S_::LDS];
  uint16_t* const ss = reinterpret_cast<uint16_t*>(smem);                          // [64][SA]
  uint16_t* const us = reinterpret_cast<uint16_t*>(smem + S_::BYTES_S);            // [2][64][SU]
  float* const red = reinterpret_cast<float*>(smem + S_::BYTES_S + 2 * S_::BYTES_U);  // [2][NW][64]
  uint16_t* const ug = reinterpret_cast<uint16_t*>(smem + S_::BYTES_S + 2 * S_::BYTES_U + S_::BYTES_RED);
  int* const active = reinterpret_cast<int*>(smem + S_::BYTES_S + 2 * S_::BYTES_U + S_::BYTES_RED +
                                             RMX_BM * S_::SG * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // XCD-aware tile order: block i runs on XCD i % 8; XCD x takes the x-th
  // contiguous range of (token, row tile) pairs
  const int rt_n = (a.B + RMX_BM - 1) / RMX_BM;
  const int ntile = a.T * rt_n;
  int lin = blockIdx.x;
  if ((ntile & 7) == 0) lin = (blockIdx.x & 7) * (ntile >> 3) + (blockIdx.x >> 3);
  const int t = lin / rt_n;
  const int64_t b0 = (int64_t)(lin - t * rt_n) * RMX_BM;

  // ---- prologue: S rows into LDS -------------------------------------------
  {
    const int c0 = lane * EPL;
    float g[EPL], be[EPL];
    if constexpr (FUSED) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        g[i] = a.g1[c0 + i];
        be[i] = a.be1[c0 + i];
      }
    }
#pragma unroll
    for (int i0 = 0; i0 < RPW; i0 += 4) {
      Vec xq[4], mq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t b = b0 + w * RPW + i0 + i;
        const int64_t bb = b < a.B ? b : a.B - 1;   // rows past B: any valid row (not stored)
        xq[i] = *reinterpret_cast<const Vec*>(a.x + (bb * a.T + t) * D + c0);
        if constexpr (FUSED) mq[i] = *reinterpret_cast<const Vec*>(a.x + mix_offset<D>(bb, t, a.T, a.dh, c0));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = w * RPW + i0 + i;
        Vec o = xq[i];
        if constexpr (FUSED) o = ln1_row<D>(xq[i], mq[i], g, be, a.eps);
        *reinterpret_cast<Vec*>(&ss[r * SA + c0]) = o;
      }
    }
  }
  __syncthreads();

  if constexpr (EM > 0) {
    // router logits of the wave's 16 rows: Lt (experts x rows) = Wr^T S^T on
    // 16x16x32 MFMAs (router fragments as A, S rows as B); gates ReLU(L)
    // stored as bf16 hi | lo pairs
    const int r16 = lane & 15, q16 = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < EM / 16; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const uint4 wa = ld16(a.wr + (((size_t)t * (D / 32) + kb) * (EM / 16) + nb) * FRAG_ELEMS + lane * 8);
        const uint4 sb = *reinterpret_cast<const uint4*>(&ss[(w * 16 + r16) * SA + kb * 32 + 8 * q16]);
        acc = mfma16x16x32(as_bf16x8(wa), as_bf16x8(sb), acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = nb * 16 + 4 * q16 + v;
        const float g = fmaxf(acc[v], 0.f);
        const uint16_t gh = f2bf(g);
        ug[(w * 16 + r16) * S_::SG + e] = gh;
        ug[(w * 16 + r16) * S_::SG + EM + e] = f2bf(g - bf2f(gh));
      }
    }
    __syncthreads();
    if constexpr (ROUTE) {
      // the gates as the FFN half uses them (hi + lo), then nothing else
      for (int i = tid; i < RMX_BM * EM; i += 64 * NW) {
        const int r = i / EM, e = i - r * EM;
        const int64_t b = b0 + r;
        if (b < a.B)
          a.gates[(b * a.T + t) * EM + e] = bf2f(ug[r * S_::SG + e]) + bf2f(ug[r * S_::SG + EM + e]);
      }
      return;
    }
    if (tid < EM) {
      int any = 0;
      for (int r = 0; r < RMX_BM; ++r) any |= ug[r * S_::SG + tid] | ug[r * S_::SG + EM + tid];
      active[tid] = any != 0;
    }
    __syncthreads();
  }

  const int KB1 = D / 16;                                   // K fragments of a W1 column tile
  const int NE = EM > 0 ? EM : 1;                           // experts of the token
  const int HE = EM > 0 ? a.h_e : a.hidden;                 // hidden units per expert
  const int KB2 = HE / 16;                                  // K fragments of one expert's W2 column tile
  const uint16_t* const w1t = a.w1 + (size_t)t * (a.hidden / 32) * KB1 * FRAG_ELEMS;
  const uint16_t* const b1t = a.b1 + (size_t)t * a.hidden;

  f32x16 acc2[2][NT2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < NT2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc2[m][j][v] = 0.f;

  const int nchunks = a.hidden / HC;
  // W1 fragments of GEMM1 group (chunk c, K steps k0 .. k0 + 15) of this wave
  auto w1frag = [&](int c, int k) {
    return ld16(w1t + ((size_t)(c * NW + w) * KB1 + k) * FRAG_ELEMS + lane * 8);
  };
  uint4 wf1[16];   // the next GEMM1 group
  // D = 256 without experts: the first half of a chunk's W1 group is loaded
  // during the previous chunk's GEMM2 (32 registers; the whole group, 64,
  // costs more than it hides), the second half at the chunk's top
  constexpr bool HALF_PF = D <= 256 && EM == 0;
  if constexpr (D > 256) {
#pragma unroll
    for (int i = 0; i < 16; ++i) wf1[i] = w1frag(0, i);
  }
  if constexpr (HALF_PF) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wf1[i] = w1frag(0, i);
  }
  int ex = 0;   // chunks run so far: the hidden buffer alternates with it
  for (int c = 0; c < nchunks; ++c) {
    // expert of this chunk (hidden units [128 c, 128 c + 128) of the token's
    // experts laid end to end); a chunk whose expert no row of the tile
    // activates is skipped by the whole workgroup
    const int je = EM > 0 ? (c * HC) / HE : 0;
    if constexpr (EM > 0) {
      if (!active[je]) continue;
    }
    const int kl0 = (c * HC - je * HE) / 16;                // first K fragment of the chunk in its expert
    const uint16_t* const w2t = a.w2 + ((size_t)t * NE + je) * (D / 32) * KB2 * FRAG_ELEMS;
    uint16_t* const ub = us + (ex & 1) * (RMX_BM * SU);
    ++ex;
    if constexpr (HALF_PF) {
#pragma unroll
      for (int i = 8; i < 16; ++i) wf1[i] = w1frag(c, i);
    } else if constexpr (D <= 256) {
#pragma unroll
      for (int i = 0; i < 16; ++i) wf1[i] = w1frag(c, i);
    }
    // b1 of this wave's hidden units. At D = 256 issued before the W2
    // prefetch below, so that the GELU waits for them only (loads complete
    // in issue order); at D = 512 right where the GELU uses them, addressed
    // from one base (both measured faster than the alternatives)
    auto load_b1 = [&](int q) {
      return *reinterpret_cast<const uint2*>(b1t + c * HC + w * 32 + 4 * hi + 8 * q);
    };
    uint2 bq[4];
    if constexpr (D <= 256 && EM == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) bq[q] = load_b1(q);
    }
    // ---- GEMM1: hidden tile 4c + w (32 units) x 64 rows ----------------------
    f32x16 acc1[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc1[0][v] = acc1[1][v] = 0.f;
#pragma unroll
    for (int k0 = 0; k0 < KT1; k0 += 16) {
      uint4 wf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        wf[i] = wf1[i];
        if (k0 + 16 < KT1) wf1[i] = w1frag(c, k0 + 16 + i);   // compile-time condition
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kc = (k0 + i) * 16 + 8 * hi;
        const uint4 s0 = *reinterpret_cast<const uint4*>(&ss[l32 * SA + kc]);
        const uint4 s1 = *reinterpret_cast<const uint4*>(&ss[(32 + l32) * SA + kc]);
        acc1[0] = mma(wf[i], s0, acc1[0]);
        acc1[1] = mma(wf[i], s1, acc1[1]);
      }
    }
    // W2 fragments of the first GEMM2 group go out before the GELU work
    constexpr int KG = 16 / NT2;   // K steps per group of 16 fragments
    uint4 wf2[KG][NT2];
#pragma unroll
    for (int k = 0; k < KG; ++k)
#pragma unroll
      for (int j = 0; j < NT2; ++j)
        wf2[k][j] = ld16(w2t + ((size_t)(w * NT2 + j) * KB2 + kl0 + k) * FRAG_ELEMS + lane * 8);
    // ---- bias + GELU, rounded hidden chunk into LDS --------------------------
    // lane holds hidden units 8q + 4 hi + r (q, r < 4) of rows l32 and 32 + l32
    {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float bias[4];
        if constexpr (D <= 256 && EM == 0) {
          unpack_row<4>(bq[q], bias);
        } else {
          const int hb = c * HC + w * 32 + 4 * hi;
          const uint2 bv = *reinterpret_cast<const uint2*>(b1t + hb + 8 * q);
          unpack_row<4>(bv, bias);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // the row's gate of this chunk's expert scales the hidden (1 for the
          // plain FFN); the gated value is what gets rounded
          float gm = 1.f;
          if constexpr (EM > 0)
            gm = bf2f(ug[(m * 32 + l32) * S_::SG + je]) + bf2f(ug[(m * 32 + l32) * S_::SG + EM + je]);
          uint2 o;
          o.x = pack_bf16x2(gm * gelu_erf(acc1[m][4 * q] + bias[0]), gm * gelu_erf(acc1[m][4 * q + 1] + bias[1]));
          o.y = pack_bf16x2(gm * gelu_erf(acc1[m][4 * q + 2] + bias[2]), gm * gelu_erf(acc1[m][4 * q + 3] + bias[3]));
          *reinterpret_cast<uint2*>(&ub[(m * 32 + l32) * SU + w * 32 + 8 * q + 4 * hi]) = o;
        }
      }
    }
    __syncthreads();
    // the next chunk's first W1 group goes out ahead of GEMM2 at D = 512 (one
    // workgroup per CU, registers to spare); at D = 256 (two per CU) at the
    // top of the next chunk: 64 more live registers through GEMM2 cost more
    // than the latency they hide. The last chunk reloads its own group: an
    // unconditional load keeps the wait counts straight.
    if constexpr (D > 256) {
      const int cn = c + 1 < nchunks ? c + 1 : c;
#pragma unroll
      for (int i = 0; i < 16; ++i) wf1[i] = w1frag(cn, i);
    }
    if constexpr (HALF_PF) {
      const int cn = c + 1 < nchunks ? c + 1 : c;
#pragma unroll
      for (int i = 0; i < 8; ++i) wf1[i] = w1frag(cn, i);
    }
    // ---- GEMM2: output column tiles w*NT2 + j, K = this chunk ----------------
#pragma unroll
    for (int k0 = 0; k0 < KT2; k0 += KG) {
      uint4 wf[KG][NT2];
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int j = 0; j < NT2; ++j) {
          wf[k][j] = wf2[k][j];
          if (k0 + KG < KT2)   // the next group's fragments (compile-time condition)
            wf2[k][j] = ld16(w2t + ((size_t)(w * NT2 + j) * KB2 + kl0 + k0 + KG + k) * FRAG_ELEMS + lane * 8);
        }
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const int kc = (k0 + k) * 16 + 8 * hi;
        const uint4 u0 = *reinterpret_cast<const uint4*>(&ub[l32 * SU + kc]);
        const uint4 u1 = *reinterpret_cast<const uint4*>(&ub[(32 + l32) * SU + kc]);
#pragma unroll
        for (int j = 0; j < NT2; ++j) {
          acc2[0][j] = mma(wf[k][j], u0, acc2[0][j]);
          acc2[1][j] = mma(wf[k][j], u1, acc2[1][j]);
        }
      }
    }
    // the next chunk writes the other hidden buffer; the barrier after that
    // write orders this chunk's reads before the buffer is written again
  }

  if constexpr (EM > 0) {
    // the experts' second biases, each scaled by its gate: one more GEMM2
    // step with the gates (hi | lo halves as 2 EM K rows) as the hidden and
    // the biases, stacked twice, as W2
#pragma unroll
    for (int k = 0; k < 2 * EM / 16; ++k) {
      const uint4 u0 = *reinterpret_cast<const uint4*>(&ug[l32 * S_::SG + k * 16 + 8 * hi]);
      const uint4 u1 = *reinterpret_cast<const uint4*>(&ug[(32 + l32) * S_::SG + k * 16 + 8 * hi]);
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        const uint4 bf =
            ld16(a.b2 + (((size_t)t * (D / 32) + w * NT2 + j) * (2 * EM / 16) + k) * FRAG_ELEMS + lane * 8);
        acc2[0][j] = mma(bf, u0, acc2[0][j]);
        acc2[1][j] = mma(bf, u1, acc2[1][j]);
      }
    }
  }

  // ---- epilogue: y = acc + b2 + S; LayerNorm; rho -----------------------------
  // lane holds columns col(j, q) + r, col = 32 (w NT2 + j) + 8q + 4 hi, rows
  // l32 (m = 0) and 32 + l32 (m = 1)
  const uint16_t* const b2t = a.b2 + (size_t)t * D;
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NT2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = 32 * (w * NT2 + j) + 8 * q + 4 * hi;
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (EM == 0) unpack_row<4>(*reinterpret_cast<const uint2*>(b2t + col), bias);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float sv[4];
        unpack_row<4>(*reinterpret_cast<const uint2*>(&ss[(m * 32 + l32) * SA + col]), sv);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y = acc2[m][j][4 * q + r] + bias[r] + sv[r];
          acc2[m][j][4 * q + r] = y;
          part[m] += y;
        }
      }
    }
  float mean[2], rstd[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float p = part[m] + __shfl_xor(part[m], 32, 64);
      if (hi == 0) red[(pass * NW + w) * RMX_BM + m * 32 + l32] = p;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* rr = red + pass * NW * RMX_BM + m * 32 + l32;
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += rr[ww * RMX_BM];
      if (pass == 0) {
        mean[m] = tot * (1.0f / D);
      } else {
        rstd[m] = 1.0f / sqrtf(tot * (1.0f / D) + a.eps);
      }
    }
    if (pass == 0) {
      part[0] = part[1] = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < NT2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float d = acc2[m][j][v] - mean[m];
            part[m] += d * d;
          }
    }
  }
  // every wave has read S (first pass above) before the second barrier, so the
  // S area now takes the output tile
#pragma unroll
  for (int j = 0; j < NT2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = 32 * (w * NT2 + j) + 8 * q + 4 * hi;
      const float4 g = *reinterpret_cast<const float4*>(a.g2 + col);
      const float4 be = *reinterpret_cast<const float4*>(a.be2 + col);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float y[4] = {acc2[m][j][4 * q], acc2[m][j][4 * q + 1], acc2[m][j][4 * q + 2], acc2[m][j][4 * q + 3]};
        uint2 o;
        o.x = pack_bf16x2((y[0] - mean[m]) * rstd[m] * g.x + be.x, (y[1] - mean[m]) * rstd[m] * g.y + be.y);
        o.y = pack_bf16x2((y[2] - mean[m]) * rstd[m] * g.z + be.z, (y[3] - mean[m]) * rstd[m] * g.w + be.w);
        *reinterpret_cast<uint2*>(&ss[(m * 32 + l32) * SA + col]) = o;
      }
    }
  __syncthreads();
  constexpr int SEG = D / 8;
  for (int i = tid; i < RMX_BM * SEG; i += 64 * NW) {
    const int r = i / SEG, sg = i - r * SEG;
    const int64_t b = b0 + r;
    if (b < a.B)
      *reinterpret_cast<uint4*>(a.out + (b * a.T + t) * D + sg * 8) =
          *reinterpret_cast<const uint4*>(&ss[r * SA + sg * 8]);
  }
}

template <int D, int EM>
void launch_block(const RmxArgs& a, int part, hipStream_t s) {
  const int tiles = a.T * ((a.B + RMX_BM - 1) / RMX_BM);
  if (part == 3) {   // router only (the host allows it for expert contexts)
    if constexpr (EM > 0)
      hipLaunchKernelGGL((rmx_block_kernel<D, false, EM, true>), dim3(tiles), dim3(64 * rmx_waves(D)), 0, s, a);
  } else if (part == 1)
    hipLaunchKernelGGL((rmx_block_kernel<D, false, EM>), dim3(tiles), dim3(64 * rmx_waves(D)), 0, s, a);
  else
    hipLaunchKernelGGL((rmx_block_kernel<D, true, EM>), dim3(tiles), dim3(64 * rmx_waves(D)), 0, s, a);
}

template <int D>
hipError_t launch_d(const RmxArgs& a, int part, hipStream_t s) {
  if (part == 0) {
    const int64_t rows = (int64_t)a.B * a.T;
    hipLaunchKernelGGL(rmx_ln1_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  } else if (a.E == 0) {
    launch_block<D, 0>(a, part, s);
  } else if constexpr (D == 256) {
    if (a.E == 16)
      launch_block<D, 16>(a, part, s);
    else if (a.E == 32)
      launch_block<D, 32>(a, part, s);
    else
      return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool rmx_width_supported(int D) { return D == 256 || D == 512; }
int rmx_hidden_multiple(int D) { return rmx_chunk(D); }
bool rmx_experts_supported(int D, int E, int h_e) { return D == 256 && (E == 16 || E == 32) && h_e % RMX_HC == 0; }

hipError_t launch_rmx(const RmxArgs& a, int part, hipStream_t s) {
  switch (a.D) {
    case 256: return launch_d<256>(a, part, s);
    case 512: return launch_d<512>(a, part, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tmx
