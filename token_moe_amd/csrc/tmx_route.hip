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
// 16 x E logits are transposed through LDS for the per-row selection.
// ---------------------------------------------------------------------------
constexpr int RT_WAVES = 4;

template <int W>
__global__ __launch_bounds__(64 * RT_WAVES) void norm_route_kernel(const RouteArgs a) {
  constexpr int KB = W / 32;
  constexpr int EMAX = 64;
  __shared__ float lg_s[RT_WAVES][16][EMAX + 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int tiles = (a.B + 16 * RT_WAVES - 1) / (16 * RT_WAVES);
  const int p = blockIdx.x / tiles;
  const int row = (blockIdx.x % tiles) * 16 * RT_WAVES + wave * 16 + l16;
  const bool valid = row < a.B;

  uint4 xr[KB];
  float ss = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    xr[kb] = valid ? ldg16(a.x + a.map.offset(row, p, kb * 32 + q * 8)) : make_uint4(0, 0, 0, 0);
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

  const int NBE = a.E / 16;
  f32x4 lg[EMAX / 16];
#pragma unroll
  for (int j = 0; j < EMAX / 16; ++j) lg[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wr = a.wr + (size_t)p * KB * NBE * FRAG_ELEMS;

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    uint16_t* h = reinterpret_cast<uint16_t*>(&xr[kb]);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = f2bf(bf2f(h[i]) * rinv * a.gain[kb * 32 + q * 8 + i]);
    if (valid && a.xhat)
      *reinterpret_cast<uint4*>(a.xhat + ((size_t)p * a.B + row) * W + kb * 32 + q * 8) = xr[kb];
    const bf16x8 af = as_bf16x8(xr[kb]);
#pragma unroll
    for (int j = 0; j < EMAX / 16; ++j)
      if (j < NBE) lg[j] = mfma16x16x32(af, as_bf16x8(ldg16(wr + ((size_t)kb * NBE + j) * FRAG_ELEMS + lane * 8)), lg[j]);
  }

  // C layout: lane holds logits[row 4q+v][expert 16j + l16]
#pragma unroll
  for (int j = 0; j < EMAX / 16; ++j)
    if (j < NBE)
#pragma unroll
      for (int v = 0; v < 4; ++v) lg_s[wave][q * 4 + v][j * 16 + l16] = lg[j][v];
  __syncthreads();

  if (q == 0 && valid) {
    const float* l = lg_s[wave][l16];
    float m = l[0];
    for (int e = 1; e < a.E; ++e) m = fmaxf(m, l[e]);
    float den = 0.f;
    for (int e = 0; e < a.E; ++e) den += expf(l[e] - m);
    uint64_t taken = 0;
    const size_t o = ((size_t)row * a.P + p) * a.top_k;
    for (int s = 0; s < a.top_k; ++s) {
      int be = -1;
      float bl = 0.f;
      for (int e = 0; e < a.E; ++e) {
        if ((taken >> e) & 1ull) continue;
        if (be < 0 || l[e] > bl) {  // strict: ties keep the lower index
          be = e;
          bl = l[e];
        }
      }
      taken |= 1ull << be;
      a.idx[o + s] = be;
      a.gate[o + s] = a.alpha * (expf(bl - m) / den);
    }
  }
}

// ---------------------------------------------------------------------------
// bucket: MoEPermute of the TokenMixer-Large systems section (2.5.1) --
// rows reordered from batch-first to expert-first.  One workgroup per
// position.  Thread t owns a contiguous run of batch rows; per-(expert,
// thread) counts are scanned in (expert, thread) order, so every expert's
// list is in ascending batch order (stable, deterministic).  Also emits the
// tile list (expert, start, count) the grouped MLP walks.
// ---------------------------------------------------------------------------
constexpr int BK_NT = 256;
constexpr int BK_EMAX = 64;

__global__ __launch_bounds__(BK_NT) void bucket_kernel(const BucketArgs a) {
  __shared__ int cnt[BK_EMAX * BK_NT];
  __shared__ int part_s[BK_NT];
  __shared__ int tstart[BK_EMAX + 1];
  const int t = threadIdx.x;
  const int p = blockIdx.x;
  const int E = a.E, k = a.top_k;
  const int chunk = (a.B + BK_NT - 1) / BK_NT;
  const int b0 = min(a.B, t * chunk), b1 = min(a.B, b0 + chunk);

  // the routed MLP launched next takes its tiles from these queues
  if (p == 0 && t < 8) a.qhead[t] = 0;
  for (int e = 0; e < E; ++e) cnt[e * BK_NT + t] = 0;
  for (int b = b0; b < b1; ++b)
    for (int s = 0; s < k; ++s) cnt[a.idx[((size_t)b * a.P + p) * k + s] * BK_NT + t] += 1;
  __syncthreads();

  // exclusive scan over the flattened (expert, thread) array; thread t owns
  // the E consecutive entries [t*E, (t+1)*E)
  int local = 0;
  for (int i = 0; i < E; ++i) local += cnt[t * E + i];
  part_s[t] = local;
  __syncthreads();
  for (int off = 1; off < BK_NT; off <<= 1) {
    const int v = (t >= off) ? part_s[t - off] : 0;
    __syncthreads();
    part_s[t] += v;
    __syncthreads();
  }
  int run = part_s[t] - local;
  for (int i = 0; i < E; ++i) {
    const int c = cnt[t * E + i];
    cnt[t * E + i] = run;
    run += c;
  }
  __syncthreads();

  int* rows = a.rows + (size_t)p * a.B * k;
  for (int b = b0; b < b1; ++b)
    for (int s = 0; s < k; ++s) {
      const int e = a.idx[((size_t)b * a.P + p) * k + s];
      const int pos = cnt[e * BK_NT + t]++;
      rows[pos] = b * k + s;
    }
  __syncthreads();

  // counts and tiles (cnt[e*NT + NT-1] now holds the end of expert e)
  if (t == 0) {
    int nt = 0;
    for (int e = 0; e < E; ++e) {
      tstart[e] = nt;
      const int beg = (e == 0) ? 0 : cnt[(e - 1) * BK_NT + BK_NT - 1];
      const int end = cnt[e * BK_NT + BK_NT - 1];
      nt += (end - beg + a.bm - 1) / a.bm;
    }
    tstart[E] = nt;
    a.ntiles[p] = nt;
  }
  __syncthreads();
  if (t < E) {
    const int e = t;
    const int beg = (e == 0) ? 0 : cnt[(e - 1) * BK_NT + BK_NT - 1];
    const int end = cnt[e * BK_NT + BK_NT - 1];
    a.counts[(size_t)p * E + e] = end - beg;
    int4* tl = a.tiles + (size_t)p * a.max_tiles;
    int j = tstart[e];
    for (int s0 = beg; s0 < end; s0 += a.bm) tl[j++] = make_int4(e, s0, min(a.bm, end - s0), 0);
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
    else
      f = ((int64_t)g * KB + kb) * NB + nb;
    dst[f * FRAG_ELEMS + lane * 8 + e] = src[i];
  }
}

// ---------------------------------------------------------------------------
// permute: Mix (inverse = 0) / Revert (inverse = 1) with the sub-layer
// kernels' RowMap (TokenMixer-Large Eq. 9-11, 13-15).
// ---------------------------------------------------------------------------
template <typename TE>
__global__ void permute_kernel(const TE* __restrict__ in, TE* __restrict__ out, int B, int T, int D, int H,
                               int inverse) {
  RowMap m{T, D, D / H, 1};
  const int W = T * (D / H);
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
}

template <int W>
hipError_t launch_route_w(const RouteArgs& a, hipStream_t s) {
  const int tiles = (a.B + 16 * RT_WAVES - 1) / (16 * RT_WAVES);
  hipLaunchKernelGGL((norm_route_kernel<W>), dim3(a.P * tiles), dim3(64 * RT_WAVES), 0, s, a);
  return hipGetLastError();
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
  hipLaunchKernelGGL(bucket_kernel, dim3(a.P), dim3(BK_NT), 0, s, a);
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

hipError_t launch_permute(const void* in, void* out, int B, int T, int D, int H, int elem_bytes, int inverse,
                          hipStream_t s) {
  const int64_t total = (int64_t)B * T * D;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (elem_bytes == 2)
    hipLaunchKernelGGL((permute_kernel<uint16_t>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), B, T, D, H, inverse);
  else
    hipLaunchKernelGGL((permute_kernel<uint32_t>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out), B, T, D, H, inverse);
  return hipGetLastError();
}

}  // namespace tmx
