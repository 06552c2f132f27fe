// tmx_route.hip -- MoE front half on gfx950: RMSNorm + router + top-k, and
// the bucket / scatter of rows per (position, expert); plus the weight
// fragment packer and the debug permutation.
#include "tmx_internal.h"

namespace tmx {

namespace {

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------------------
// norm_route: one wave per 16 rows of one position.
//
// Sparse-Pertoken MoE router (TokenMixer-Large Eq. 19 and 21): the rows are
// RMS-normalised (section 2.3.3) and rounded to bf16 -- the same x_hat the
// experts consume, also written to the x_hat buffer -- then
//   logits = x_hat @ Wr_p          (bf16 MFMA, fp32 accumulate)
//   pi     = softmax(logits) over all E
//   chosen = top_k experts by (largest logit, then lowest index)
//   gate   = alpha * pi[chosen]     (not renormalised)
// Each lane holds its rows' elements directly in the MFMA A-fragment layout
// (row l%16, k = 32*kb + 8*(l/16) + i), so x_hat never goes through LDS; the
// selection runs on the MFMA output layout with cross-lane reductions. The
// workgroup (128 rows of one position) also counts its choices per expert
// for the bucket kernel.
// ---------------------------------------------------------------------------
// 8 waves (128 rows) per workgroup: the position's router fragments are
// staged into LDS once per 128 rows, and at 128 VGPRs four waves share each
// SIMD (two workgroups per CU); measured on the large MoE stack against 4
// waves: 0.304 -> 0.263 ms (Mix sub-layer), 0.266 -> 0.225 ms (Revert);
// 16 waves (one workgroup per CU) was slower
constexpr int RT_WAVES = 8;

// 16-lane butterflies on DPP (one DPP row = 16 lanes = the lanes holding one
// row's logits): quad xor 1, quad xor 2, half-row mirror, row mirror leave
// the reduction of all 16 lanes in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_QXOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QXOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_HMIRROR = 0x141; // row_half_mirror
constexpr int DPP_MIRROR = 0x140;  // row_mirror

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QXOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QXOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HMIRROR>(v));
  return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QXOR1>(v);
  v += dpp_f<DPP_QXOR2>(v);
  v += dpp_f<DPP_HMIRROR>(v);
  return v + dpp_f<DPP_MIRROR>(v);
}
// (value, index) maximum: larger value, lower index on ties
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = dpp_f<CTRL>(bv);
  const int oe = dpp_i<CTRL>(be);
  if (ov > bv || (ov == bv && oe < be)) {
    bv = ov;
    be = oe;
  }
}
__device__ __forceinline__ void row16_argmax(float& bv, int& be) {
  argmax_step<DPP_QXOR1>(bv, be);
  argmax_step<DPP_QXOR2>(bv, be);
  argmax_step<DPP_HMIRROR>(bv, be);
  argmax_step<DPP_MIRROR>(bv, be);
}

// E4M3 codes of the 8 bf16 values in w times 2^-k (exact), clamped to +-448
// first (the conversion rounds to nearest even but does not saturate)
__device__ __forceinline__ uint32_t e4m3x4_bf16(uint32_t v0, uint32_t v1, float sc) {
  const float x0 = fminf(fmaxf(__uint_as_float(v0 << 16) * sc, -448.f), 448.f);
  const float x1 = fminf(fmaxf(__uint_as_float(v0 & 0xFFFF0000u) * sc, -448.f), 448.f);
  const float x2 = fminf(fmaxf(__uint_as_float(v1 << 16) * sc, -448.f), 448.f);
  const float x3 = fminf(fmaxf(__uint_as_float(v1 & 0xFFFF0000u) * sc, -448.f), 448.f);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}
__device__ __forceinline__ uint2 e4m3x8_bf16(const uint4& w, float sc) {
  return make_uint2(e4m3x4_bf16(w.x, w.y, sc), e4m3x4_bf16(w.z, w.w, sc));
}
// largest magnitude among the 8 bf16 values of w, as its bf16 bit pattern
// (magnitudes order as their 15-bit patterns)
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const uint4& w) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = v[i] & 0x7FFFu, hi = (v[i] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// XQ8: also write the MXFP8 copy of x_hat (a.xq8, a.xe8); a compile-time
// switch, so the bf16 router carries none of its code or registers
// (the MXFP8 instantiations are held to four waves per SIMD, 128 VGPRs: they
// spill a few dozen registers at W = 768 but run 3-6% faster than at two
// waves per SIMD; the bf16 ones reach four waves unconstrained)
template <int W, int NBE, bool XQ8>
__global__ __launch_bounds__(64 * RT_WAVES, XQ8 ? 4 : 2) void norm_route_kernel(const RouteArgs a) {
  constexpr int KB = W / 32;
  constexpr int EMAX = 64;
  constexpr int NFR = KB * NBE;              // router fragments of one position
  __shared__ int hist_s[EMAX];
  __shared__ __attribute__((aligned(16))) uint16_t wr_s[NFR * FRAG_ELEMS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int tiles = (a.B + 16 * RT_WAVES - 1) / (16 * RT_WAVES);
  const int p = blockIdx.x / tiles;
  const int chunk = blockIdx.x % tiles;
  const int row = chunk * 16 * RT_WAVES + wave * 16 + l16;
  const bool valid = row < a.B;
  if (a.hist)
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) hist_s[e] = 0;
  // row and position parts of this lane's offsets, and its 8-column runs
  // (k-blocks of 32 columns, the lane's quarter q) through the map's column
  // cursor, so the Mix map's division by D/H is stepped through instead of
  // repeated
  const int64_t rbase = a.map.row(valid ? row : 0) + a.map.pos(p);
  uint4 xr[KB];
  float ss = 0.f;
  {
    RowMap::Cursor cur = a.map.cursor(q * 8);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      xr[kb] = valid ? ldg16(a.x + rbase + cur.col()) : make_uint4(0, 0, 0, 0);
      cur.advance(32);
    }
  }
  // the position's router fragments, staged once for the eight waves (L2
  // hits after the first workgroup of a position; issued after the row
  // loads so that those are already in flight)
  {
    const uint16_t* src = a.wr + (size_t)p * NFR * FRAG_ELEMS;
    for (int i = threadIdx.x * 8; i < NFR * FRAG_ELEMS; i += 64 * RT_WAVES * 8)
      *reinterpret_cast<uint4*>(&wr_s[i]) = ldg16(src + i);
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(&xr[kb]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = bf2f(h[i]);
      ss += f * f;
    }
  }
  // the four lanes l16, l16+16, l16+32, l16+48 hold one row
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  const float rinv = 1.0f / sqrtf(ss / (float)W + a.eps);
  __syncthreads();                           // router fragments staged
  // the rows stay packed between the two passes: without this fence the
  // compiler keeps the first pass's fp32 copies (2 registers per element)
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(xr[kb].x), "+v"(xr[kb].y), "+v"(xr[kb].z), "+v"(xr[kb].w));

  f32x4 lg[NBE];
#pragma unroll
  for (int j = 0; j < NBE; ++j) lg[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wr = wr_s + lane * 8;
  // MXFP8 copy of the rows (xq8): exponent bytes of the row's 32-column
  // blocks, packed 4 to a dword (every lane of the row holds all of them)
  uint32_t eb[KB / 4] = {};

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(&xr[kb]);
    const float4 g0 = *reinterpret_cast<const float4*>(a.gain + kb * 32 + q * 8);
    const float4 g1 = *reinterpret_cast<const float4*>(a.gain + kb * 32 + q * 8 + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float n[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) n[i] = bf2f(h[i]) * rinv * gv[i];
    // round to nearest even (v_cvt_pk_bf16_f32)
    xr[kb].x = pack_bf16x2(n[0], n[1]);
    xr[kb].y = pack_bf16x2(n[2], n[3]);
    xr[kb].z = pack_bf16x2(n[4], n[5]);
    xr[kb].w = pack_bf16x2(n[6], n[7]);
    if (valid && a.xhat)
      *reinterpret_cast<uint4*>(a.xhat + ((size_t)p * a.B + row) * W + kb * 32 + q * 8) = xr[kb];
    if constexpr (XQ8) {
      // the bf16 row quantised per 32-column block (this lane's 8 columns and
      // those of lanes ^ 16, ^ 32, ^ 48): exponent floor(log2(amax)) - 8
      uint32_t mb = bf16x8_absmax_bits(xr[kb]);
      const uint32_t m16 = (uint32_t)__shfl_xor((int)mb, 16, 64);
      mb = mb > m16 ? mb : m16;
      const uint32_t m32 = (uint32_t)__shfl_xor((int)mb, 32, 64);
      mb = mb > m32 ? mb : m32;
      const float amax = __uint_as_float(mb << 16);
      int e = 0;
      (void)frexpf(amax, &e);
      int k = amax > 0.f ? e - 9 : -127;
      k = k < -127 ? -127 : (k > 127 ? 127 : k);
      const uint2 c = e4m3x8_bf16(xr[kb], ldexpf(1.f, -k));
      if (valid) *reinterpret_cast<uint2*>(a.xq8 + ((size_t)p * a.B + row) * W + kb * 32 + q * 8) = c;
      eb[kb / 4] |= (uint32_t)(k + 127) << (8 * (kb % 4));
    }
    const bf16x8 af = as_bf16x8(xr[kb]);
#pragma unroll
    for (int j = 0; j < NBE; ++j)
      lg[j] = mfma16x16x32(af, as_bf16x8(*reinterpret_cast<const uint4*>(wr + (kb * NBE + j) * FRAG_ELEMS)), lg[j]);
  }

  if (XQ8 && valid) {
    static_assert(KB % 4 == 0, "exponent dwords");
    uint32_t* er = reinterpret_cast<uint32_t*>(a.xe8 + ((size_t)p * a.B + row) * KB);
#pragma unroll
    for (int d = 0; d < KB / 4; ++d)
      if ((d & 3) == q) er[d] = eb[d];
  }

  // Softmax and top-k per row. C layout: lane (l16, q) holds the logits of
  // rows 4q+v (v = 0..3) for experts 16j + l16, so a row's E logits sit in
  // the 16 lanes of one DPP row and every reduction is a 16-lane butterfly.
  // Selection key: larger logit first, the lower expert index on ties.
  const int rb0 = chunk * 16 * RT_WAVES + wave * 16 + 4 * q;
  // the lane's four rows are independent: every step below runs on all four
  // at once, so each DPP butterfly has four chains to interleave
  float m[4], den[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    m[v] = lg[0][v];
#pragma unroll
    for (int j = 1; j < NBE; ++j) m[v] = fmaxf(m[v], lg[j][v]);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) m[v] = row16_max(m[v]);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    den[v] = 0.f;
#pragma unroll
    for (int j = 0; j < NBE; ++j) den[v] += expf(lg[j][v] - m[v]);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) den[v] = row16_sum(den[v]);
  uint32_t taken[4] = {0u, 0u, 0u, 0u};
  for (int s = 0; s < a.top_k; ++s) {
    float bv[4];
    int be[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      bv[v] = -INFINITY;
      be[v] = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < NBE; ++j) {
        // a NaN logit (a non-finite input row) ranks as -inf, and the lane's
        // first untaken expert is always a candidate: every slot then names a
        // distinct expert in [0, E) whatever the row holds
        const float l = lg[j][v] == lg[j][v] ? lg[j][v] : -INFINITY;
        if (!((taken[v] >> j) & 1u) && (be[v] == 0x7fffffff || l > bv[v])) {   // j ascending: ties keep the lower index
          bv[v] = l;
          be[v] = 16 * j + l16;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) row16_argmax(bv[v], be[v]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if ((be[v] & 15) == l16) taken[v] |= 1u << (be[v] >> 4);
      const int r = rb0 + v;
      if (r < a.B && l16 == (s & 15)) {
        const size_t o = ((size_t)r * a.P + p) * a.top_k + s;
        a.idx[o] = be[v];
        a.gate[o] = a.alpha * (expf(bv[v] - m[v]) / den[v]);
        if (a.hist) atomicAdd(&hist_s[be[v]], 1);
      }
    }
  }
  if (a.hist) {
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += blockDim.x)
      a.hist[((size_t)p * tiles + chunk) * a.E + e] = hist_s[e];
  }
}

// ---------------------------------------------------------------------------
// bucket: MoEPermute of the TokenMixer-Large systems section (2.5.1) --
// rows reordered from batch-first to expert-first. One workgroup per
// (position, 128-row chunk): from the router's per-chunk expert counts it
// takes the start of its chunk's entries in every expert list, then places
// its entries in (row, slot) order with wave ballots, so every list is in
// ascending (batch row, slot) order (stable, deterministic). Workgroup
// (p, 0) also emits the tile list (expert, start, count) the grouped MLP
// walks and the per-expert counts.
// ---------------------------------------------------------------------------
constexpr int BK_NT = 256;
constexpr int BK_EMAX = 64;
constexpr int BK_ROWS = 16 * RT_WAVES;   // rows per chunk, as counted by norm_route
static_assert(BK_ROWS >= 64, "the host sizes the per-chunk counts for chunks of at least 64 rows");

__global__ __launch_bounds__(BK_NT) void bucket_kernel(const BucketArgs a) {
  __shared__ int base_s[BK_EMAX];          // start of this chunk's entries per expert
  __shared__ int tot_s[BK_EMAX];
  __shared__ int wcnt[BK_NT / 64][BK_EMAX];
  __shared__ int run_s[BK_EMAX];
  __shared__ int gtot[BK_NT / 16][BK_EMAX];   // per chunk-group partial counts (E >= 16)
  __shared__ int gpre[BK_NT / 16][BK_EMAX];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int E = a.E, k = a.top_k;
  const int C = (a.B + BK_ROWS - 1) / BK_ROWS;
  const int p = blockIdx.x / C, c = blockIdx.x % C;
  // the routed MLP launched next takes its tiles from these queues
  if (blockIdx.x == 0 && t < 8) a.qhead[t] = 0;

  // chunk counts of the position: thread (group g, expert e) sums chunks
  // g, g + G, ...; the G partial sums per expert are then added in LDS
  {
    const int G = BK_NT / E;
    const int e = t % E, g = t / E;
    int tot = 0, pre = 0;
    if (g < G) {
      const int* h = a.hist + (size_t)p * C * E + e;
      // unrolled so that the loads of one thread are in flight together
#pragma unroll 8
      for (int cc = g; cc < C; cc += G) {
        const int n = h[(size_t)cc * E];
        tot += n;
        if (cc < c) pre += n;
      }
      gtot[g][e] = tot;
      gpre[g][e] = pre;
    }
  }
  __syncthreads();
  if (t < E) {
    int tot = 0, pre = 0;
    for (int g = 0; g < BK_NT / E; ++g) {
      tot += gtot[g][t];
      pre += gpre[g][t];
    }
    tot_s[t] = tot;
    base_s[t] = pre;
    run_s[t] = 0;
  }
  __syncthreads();
  if (t == 0) {
    int off = 0;
    for (int e = 0; e < E; ++e) {
      base_s[e] += off;
      off += tot_s[e];
    }
  }
  __syncthreads();

  // tiles and counts of the position: thread e writes expert e's tiles,
  // which start after the tiles of experts 0 .. e-1
  if (c == 0) {
    __shared__ int tstart[BK_EMAX + 1];
    if (t == 0) {
      int nt = 0;
      for (int e = 0; e < E; ++e) {
        tstart[e] = nt;
        nt += (tot_s[e] + a.bm - 1) / a.bm;
      }
      tstart[E] = nt;
      a.ntiles[p] = nt;
    }
    __syncthreads();
    if (t < E) {
      const int n = tot_s[t];
      a.counts[(size_t)p * E + t] = n;
      int4* tl = a.tiles + (size_t)p * a.max_tiles + tstart[t];
      const int off = base_s[t];               // entries of experts before t (chunk 0: no prefix)
      for (int s0 = 0, j = 0; s0 < n; s0 += a.bm, ++j) tl[j] = make_int4(t, off + s0, min(a.bm, n - s0), 0);
    }
  }

  const int r0 = c * BK_ROWS;
  const int nent = min(BK_ROWS, a.B - r0) * k;
  int* rows = a.rows + (size_t)p * a.B * k;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  for (int i0 = 0; i0 < nent; i0 += BK_NT) {
    const int id = i0 + t;
    const int b = r0 + id / k, sl = id % k;
    const int e = id < nent ? a.idx[((size_t)b * a.P + p) * k + sl] : -1;
    int rank = 0;
    for (int ee = 0; ee < E; ++ee) {
      const uint64_t m = __ballot(e == ee);
      if (e == ee) rank = __popcll(m & lt);
      if (lane == 0) wcnt[wave][ee] = __popcll(m);
    }
    __syncthreads();
    if (e >= 0 && e < E) {
      int pos = base_s[e] + run_s[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      rows[pos] = b * k + sl;
    }
    __syncthreads();
    if (t < E) {
      int n = 0;
      for (int w = 0; w < BK_NT / 64; ++w) n += wcnt[w][t];
      run_s[t] += n;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// pack: row-major [G][K][N] bf16 -> MFMA B-operand fragments.
//   FRAG_16x16x32: k-block 32, n-block 16, lane = 16*(kk/8) + nn
//   FRAG_32x32x16: k-block 16, n-block 32, lane = 32*(kk/8) + nn
// element i = kk % 8 within the lane's 16 bytes.
//   layout 0: frag = ((g*NB + nb)*KB + kb)*2 + which   (gate|up interleaved)
//   layout 1: frag = (g*KB + kb)*NB + nb               (down, router)
// ---------------------------------------------------------------------------
__global__ void pack_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int G, int K,
                            int N, int layout, int which, int frag32) {
  const int64_t total = (int64_t)G * K * N;
  const int KF = frag32 ? 16 : 32, NF = frag32 ? 32 : 16;
  const int KB = K / KF, NB = N / NF;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i % N);
    const int64_t gk = i / N;
    const int k = (int)(gk % K);
    const int g = (int)(gk / K);
    const int kb = k / KF, kk = k % KF, nb = n / NF, nn = n % NF;
    const int lane = (kk >> 3) * NF + nn, e = kk & 7;
    int64_t f;
    if (layout == 0)
      f = (((int64_t)g * NB + nb) * KB + kb) * 2 + which;
    else if (layout == 1)
      f = ((int64_t)g * KB + kb) * NB + nb;
    else
      f = ((int64_t)g * NB + nb) * KB + kb;
    dst[f * FRAG_ELEMS + lane * 8 + e] = src[i];
  }
}

// MXFP8 weight packing (load time, layout in tmx_internal.h): one thread per
// (matrix, column, 32-element K-block). The block's shared exponent is
// floor(log2(amax)) - 8 (E4M3's largest normal is 1.75 * 2^8), the codes are
// the hardware's round-to-nearest-even conversion of x * 2^-k after clamping
// to +-448 (the conversion itself does not saturate).
__global__ void pack_mx_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                               uint8_t* __restrict__ rec, int G, int K, int N, int down, int which, int R) {
  const int KBLK = K / 32;
  const int64_t total = (int64_t)G * N * KBLK;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(i % KBLK);
    const int64_t gn = i / KBLK;
    const int n = (int)(gn % N);
    const int g = (int)(gn / N);
    const uint16_t* col = src + (int64_t)g * K * N + n;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      v[r] = bf2f(col[(int64_t)(b * 32 + r) * N]);
      amax = fmaxf(amax, fabsf(v[r]));
    }
    int e = 0;
    (void)frexpf(amax, &e);
    int k = amax > 0.f ? e - 1 - 8 : -127;
    k = k < -127 ? -127 : (k > 127 ? 127 : k);
    const int nb = n / 32, h0 = n % 32;
    const int half = b & 1;   // K-block within the 64-K step
    int64_t frag;
    if (!down) {
      const int KS = K / 64, NB = N / 32;
      frag = (((int64_t)g * NB + nb) * KS + (b >> 1)) * 2 + which;
    } else {
      const int KB = K / 64, NB = N / 32;
      frag = ((int64_t)g * KB + (b >> 1)) * NB + nb;
    }
#pragma unroll
    for (int r = 0; r < 32; r += 2) {
      float y0 = ldexpf(v[r], -k), y1 = ldexpf(v[r + 1], -k);
      y0 = fminf(fmaxf(y0, -448.f), 448.f);
      y1 = fminf(fmaxf(y1, -448.f), 448.f);
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      const int lane = (r / 16) * 32 + h0;
      uint8_t* d = dst + (frag * 2 + half) * 1024 + lane * 16 + (r % 16);
      d[0] = (uint8_t)(w & 0xFF);
      d[1] = (uint8_t)((w >> 8) & 0xFF);
    }
    // scale byte in the record of the lane that supplies it to the MFMA
    // (row h0, K-block parity b & 1 -> lane h0 + 32 (b & 1))
    // (chunk c of 128 hidden units, matrix m, byte q of the matrix's DW
    // dwords in that chunk; DW = W / 256 with W = K for gate/up, N for down)
    const int lane_s = h0 + 32 * (b & 1);
    int wave, c, m, q, DW;
    if (!down) {
      DW = K / 256;
      wave = nb % 4;
      c = nb / 4;
      m = which;
      q = b >> 1;
    } else {
      DW = N / 256;
      const int nbo = N / 128;   // column blocks per wave
      wave = nb / nbo;
      c = b / 4;
      m = 2;
      q = (nb % nbo) * 2 + ((b % 4) >> 1);
    }
    const int dword = (c * 3 + m) * DW + (q >> 2);
    rec[((((int64_t)g * 4 + wave) * 64 + lane_s) * R + dword) * 4 + (q & 3)] = (uint8_t)(k + 127);
  }
}

// ---------------------------------------------------------------------------
// permute: Mix (inverse = 0) / Revert (inverse = 1) of [B, T, D] <-> [B, H,
// T*D/H] (TokenMixer-Large Eq. 9-11, 13-15), through RowMap in each of the
// forms the sub-layer kernels address block-layout rows with:
//   PERM_ELEM    offset(b, p, w) per element (the fp32 path; the fused MLP's
//                per-unit form when a lane's column group changes per unit)
//   PERM_LANECOL the fused MLP's row I/O: 256 threads move 64 rows of one
//                position in 8-column units, unit u = tid + 256 i covering
//                row u / U8 and columns 8 (u % U8); when 256 % U8 == 0 a
//                lane's column part col() is computed once and its offsets
//                are row(b) + pos(p) + that part, as in the MLP kernel
//   PERM_CURSOR  the router's form: the 4 lanes l16 + 16 q of a row read its
//                8-column runs at columns 8 q + 32 kb through the column cursor
// ---------------------------------------------------------------------------
template <typename TE>
struct alignas(8 * sizeof(TE)) Vec8 {
  TE v[8];
};

template <typename TE, int FORM>
__global__ __launch_bounds__(256) void permute_kernel(const TE* __restrict__ in, TE* __restrict__ out, int B, int T,
                                                      int D, int H, int inverse) {
  const RowMap m{T, D, D / H, 1};
  const int W = T * (D / H);
  if constexpr (FORM == PERM_ELEM) {
    const int64_t total = (int64_t)B * H * W;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int w = (int)(i % W);
      const int64_t bh = i / W;
      const int h = (int)(bh % H);
      const int64_t b = bh / H;
      const int64_t o = m.offset(b, h, w);
      if (inverse)
        out[o] = in[i];
      else
        out[i] = in[o];
    }
  } else {
    // block (position h, 64-row chunk); 8-element units
    const int chunks = (B + 63) / 64;
    const int h = blockIdx.x / chunks;
    const int64_t b0 = (int64_t)(blockIdx.x % chunks) * 64;
    const int tid = threadIdx.x;
    auto move = [&](int64_t b, int w, int64_t o) {
      if (b >= B) return;
      const int64_t mi = (b * H + h) * W + w;   // mixed-layout element
      if (inverse)
        *reinterpret_cast<Vec8<TE>*>(out + o) = *reinterpret_cast<const Vec8<TE>*>(in + mi);
      else
        *reinterpret_cast<Vec8<TE>*>(out + mi) = *reinterpret_cast<const Vec8<TE>*>(in + o);
    };
    if constexpr (FORM == PERM_LANECOL) {
      const int U8 = W / 8;
      if (256 % U8 == 0) {
        const int lcol = m.col((tid % U8) * 8);
        for (int r = tid / U8; r < 64; r += 256 / U8) move(b0 + r, (tid % U8) * 8, m.row(b0 + r) + m.pos(h) + lcol);
      } else {
        for (int u = tid; u < 64 * U8; u += 256) {
          const int r = u / U8, c8 = u - r * U8;
          move(b0 + r, c8 * 8, m.offset(b0 + r, h, c8 * 8));
        }
      }
    } else {
      const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, q = lane >> 4;
      const int64_t b = b0 + wave * 16 + l16;
      const int64_t rbase = m.row(b < B ? b : 0) + m.pos(h);
      RowMap::Cursor cur = m.cursor(q * 8);
      for (int kb = 0; kb < W / 32; ++kb) {
        move(b, kb * 32 + q * 8, rbase + cur.col());
        cur.advance(32);
      }
    }
  }
}

template <int W, int NBE>
hipError_t launch_route_wn(const RouteArgs& a, hipStream_t s) {
  const int tiles = (a.B + 16 * RT_WAVES - 1) / (16 * RT_WAVES);
  if (a.xq8) {
    // the MXFP8 copy exists for the MXFP8 MoE widths only
    if constexpr (W == 512 || W == 768)
      hipLaunchKernelGGL((norm_route_kernel<W, NBE, true>), dim3(a.P * tiles), dim3(64 * RT_WAVES), 0, s, a);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((norm_route_kernel<W, NBE, false>), dim3(a.P * tiles), dim3(64 * RT_WAVES), 0, s, a);
  }
  return hipGetLastError();
}

template <int W>
hipError_t launch_route_w(const RouteArgs& a, hipStream_t s) {
  switch (a.E / 16) {
    case 1: return launch_route_wn<W, 1>(a, s);
    case 2: return launch_route_wn<W, 2>(a, s);
    case 3: return launch_route_wn<W, 3>(a, s);
    case 4: return launch_route_wn<W, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_norm_route(int W, const RouteArgs& a, hipStream_t s) {
  switch (W) {
    case 128: return launch_route_w<128>(a, s);
    case 256: return launch_route_w<256>(a, s);
    case 512: return launch_route_w<512>(a, s);
    case 768: return launch_route_w<768>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bucket(const BucketArgs& a, hipStream_t s) {
  const int C = (a.B + BK_ROWS - 1) / BK_ROWS;
  hipLaunchKernelGGL(bucket_kernel, dim3(a.P * C), dim3(BK_NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int G, int K, int N, int layout, int which,
                       int frag, hipStream_t s) {
  const int64_t total = (int64_t)G * K * N;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, G, K, N, layout, which,
                     frag == FRAG_32x32x16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_pack_mx(const uint16_t* src, uint8_t* dst, uint8_t* rec, int G, int K, int N, int down, int which,
                          int rec_dwords, hipStream_t s) {
  const int W = down ? N : K, hidden = down ? K : N;
  if ((W != 256 && W != 512 && W != 768) || hidden % MLP_HC != 0 || hidden > mx_max_chunks(W) * MLP_HC ||
      rec_dwords < mx_rec_dwords(W, hidden))
    return hipErrorInvalidValue;
  const int64_t total = (int64_t)G * N * (K / 32);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_mx_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, rec, G, K, N, down, which,
                     rec_dwords);
  return hipGetLastError();
}

template <typename TE, int FORM>
void launch_permute_t(const void* in, void* out, int B, int T, int D, int H, int inverse, hipStream_t s) {
  int64_t blocks;
  if (FORM == PERM_ELEM)
    blocks = std::min<int64_t>(((int64_t)B * T * D + 255) / 256, 65536);
  else
    blocks = (int64_t)H * ((B + 63) / 64);
  hipLaunchKernelGGL((permute_kernel<TE, FORM>), dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const TE*>(in),
                     static_cast<TE*>(out), B, T, D, H, inverse);
}

hipError_t launch_permute(const void* in, void* out, int B, int T, int D, int H, int elem_bytes, int inverse,
                          int form, hipStream_t s) {
  if (elem_bytes == 2) {
    if (form == PERM_ELEM) launch_permute_t<uint16_t, PERM_ELEM>(in, out, B, T, D, H, inverse, s);
    else if (form == PERM_LANECOL) launch_permute_t<uint16_t, PERM_LANECOL>(in, out, B, T, D, H, inverse, s);
    else launch_permute_t<uint16_t, PERM_CURSOR>(in, out, B, T, D, H, inverse, s);
  } else {
    if (form == PERM_ELEM) launch_permute_t<uint32_t, PERM_ELEM>(in, out, B, T, D, H, inverse, s);
    else if (form == PERM_LANECOL) launch_permute_t<uint32_t, PERM_LANECOL>(in, out, B, T, D, H, inverse, s);
    else launch_permute_t<uint32_t, PERM_CURSOR>(in, out, B, T, D, H, inverse, s);
  }
  return hipGetLastError();
}

}  // namespace tmx
