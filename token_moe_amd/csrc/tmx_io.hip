// tmx_io.hip -- the model's front and back on gfx950 bf16 MFMA:
//
//   tokenizer (TokenMixer-Large summary section 2.2, Eq. 2-4): token t of a
//     sample is MLP_t of its semantic group's concatenated embeddings (Eq. 2),
//     token 0 the global token, an MLP over all groups' embeddings (Eq. 3-4);
//     MLP(v) = ReLU(v W1) W2, no biases;
//   head (section 2.1; the tokenmixerlarge README's block diagram): the mean
//     of the T output tokens, then the projection MLP to one logit.
//
// Both follow the fused MLP's scheme: one workgroup of 4 waves owns 64 rows;
// the first GEMM computes S^T = W1^T v^T with packed weight fragments as the
// MFMA A operand and the rows (staged in LDS) as B, so a lane's accumulators
// hold 4 consecutive hidden units of one row; the rounded hidden goes to LDS
// and feeds the second GEMM (tokenizer) or a per-row dot product (head).
#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int IO_BM = 64;       // rows per workgroup
constexpr int IO_NT = 256;      // 4 waves
constexpr int IO_KS = 64;       // embedding columns per staged slab
constexpr int IO_SS = IO_KS + 8;   // slab row stride (bf16): rows on distinct bank groups

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// tokenizer: grid (T positions) x (row tiles); NH = hidden blocks of 32 per
// wave (h = 128 NH), ND = output blocks of 32 per wave (D = 128 ND)
// ---------------------------------------------------------------------------
template <int NH, int ND>
__global__ __launch_bounds__(IO_NT, 1) void tok_kernel(const IoArgs a) {
  constexpr int H = 128 * NH, D = 128 * ND;
  constexpr int US = H + 8;                       // U row stride (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t slab[2][IO_BM * IO_SS];
  __shared__ __attribute__((aligned(16))) uint16_t us[IO_BM * US];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int tiles = (a.B + IO_BM - 1) / IO_BM;
  const int t = blockIdx.x / tiles;
  const int b0 = (blockIdx.x % tiles) * IO_BM;
  const int4 pt = a.tok_pos[t];                   // (column offset, K, W1 fragment offset, 0)
  const int c0 = pt.x, K = pt.y;
  const uint16_t* w1 = a.tok_w1 + (size_t)pt.z * FRAG_ELEMS;
  const uint16_t* w2 = a.tok_w2 + (size_t)t * (H / 16) * (D / 32) * FRAG_ELEMS;
  const int KB = K / 16;

  // slab staging: 64 rows x 64 columns, 16 bytes per thread and load, two
  // loads per thread; rows past B read row B-1 and columns past the group's
  // last (the second half of a last half slab) read its last 8 columns --
  // neither is used
  auto load_slab = [&](int s, uint4* v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + i * IO_NT;              // unit: row u / 8, 8 columns (u % 8) * 8
      const int r = u >> 3, cc = (u & 7) * 8;
      const int b = min(b0 + r, a.B - 1);
      const int col = min(s * IO_KS + cc, K - 8);
      v[i] = ldg16(a.emb + (size_t)b * a.F + c0 + col);
    }
  };
  auto store_slab = [&](int buf, const uint4* v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + i * IO_NT;
      *reinterpret_cast<uint4*>(&slab[buf][(u >> 3) * IO_SS + (u & 7) * 8]) = v[i];
    }
  };

  // ---- GEMM1: S^T [H x 64] over K, slabs of 64 columns (K is a multiple of
  // 32: a last half slab runs two k-steps)
  f32x16 acc[NH][2];
#pragma unroll
  for (int j = 0; j < NH; ++j) acc[j][0] = acc[j][1] = f32x16{};
  const int nslab = (K + IO_KS - 1) / IO_KS;
  {
    uint4 v[2];
    load_slab(0, v);
    store_slab(0, v);
  }
  __syncthreads();
  for (int s = 0; s < nslab; ++s) {
    uint4 nv[2];
    const bool more = s + 1 < nslab;
    if (more) load_slab(s + 1, nv);
    const uint16_t* sb = slab[s & 1];
    const int steps = min(IO_KS, K - s * IO_KS) / 16;
    for (int q = 0; q < steps; ++q) {
      const int kb = s * (IO_KS / 16) + q;
      uint4 xb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        xb[rb] = *reinterpret_cast<const uint4*>(&sb[(rb * 32 + l32) * IO_SS + q * 16 + h32 * 8]);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        // hidden block nb = wave * NH + j; layout 2 fragment (nb, kb)
        const uint4 wf = ldg16(w1 + ((size_t)(wave * NH + j) * KB + kb) * FRAG_ELEMS + lane * 8);
        acc[j][0] = mfma32(wf, xb[0], acc[j][0]);
        acc[j][1] = mfma32(wf, xb[1], acc[j][1]);
      }
    }
    if (more) store_slab((s + 1) & 1, nv);
    __syncthreads();
  }

  // ---- U = rho(ReLU(S)) -> LDS: lane holds row rb*32 + l32, hidden units
  // 32 (wave NH + j) + 8 (v / 4) + 4 h32 + v % 4
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& c = acc[j][rb];
        uint2 w;
        w.x = pack_bf16x2(fmaxf(c[4 * g4], 0.f), fmaxf(c[4 * g4 + 1], 0.f));
        w.y = pack_bf16x2(fmaxf(c[4 * g4 + 2], 0.f), fmaxf(c[4 * g4 + 3], 0.f));
        *reinterpret_cast<uint2*>(&us[(rb * 32 + l32) * US + (wave * NH + j) * 32 + 8 * g4 + 4 * h32]) = w;
      }
  __syncthreads();

  // ---- GEMM2: O^T [D x 64] = W2^T U^T; wave owns output blocks wave ND + j
  f32x16 o[ND][2];
#pragma unroll
  for (int j = 0; j < ND; ++j) o[j][0] = o[j][1] = f32x16{};
  for (int kb = 0; kb < H / 16; ++kb) {
    uint4 ub[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      ub[rb] = *reinterpret_cast<const uint4*>(&us[(rb * 32 + l32) * US + kb * 16 + h32 * 8]);
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const uint4 wf = ldg16(w2 + ((size_t)(wave * ND + j) * (H / 16) + kb) * FRAG_ELEMS + lane * 8);
      o[j][0] = mfma32(wf, ub[0], o[j][0]);
      o[j][1] = mfma32(wf, ub[1], o[j][1]);
    }
  }

  // ---- X[b, t, :] = rho(O): 4 consecutive columns (8 bytes) per v-group
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int b = b0 + rb * 32 + l32;
    if (b >= a.B) continue;
    uint16_t* row = a.x_out + ((size_t)b * a.T + t) * D;
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& c = o[j][rb];
        uint2 w;
        w.x = pack_bf16x2(c[4 * g4], c[4 * g4 + 1]);
        w.y = pack_bf16x2(c[4 * g4 + 2], c[4 * g4 + 3]);
        *reinterpret_cast<uint2*>(row + (wave * ND + j) * 32 + 8 * g4 + 4 * h32) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// head: one workgroup per 64 rows; ND = D / 128, NH = h_head / 128
// ---------------------------------------------------------------------------
template <int ND, int NH>
__global__ __launch_bounds__(IO_NT, 1) void head_kernel(const IoArgs a) {
  constexpr int D = 128 * ND, HH = 128 * NH;
  constexpr int PS = D + 8;                       // pooled row stride (bf16)
  constexpr int U8 = D / 8;                       // 16-byte units per row
  __shared__ __attribute__((aligned(16))) uint16_t ps[IO_BM * PS];
  __shared__ float red[4][IO_BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int b0 = blockIdx.x * IO_BM;
  const float inv_t = 1.0f / (float)a.T;

  // ---- pooled rows: mean over the T tokens in fp32, rounded to bf16 once.
  // Unit u = (row u / U8, 8 columns); tokens summed in order t = 0..T-1
  for (int u = tid; u < IO_BM * U8; u += IO_NT) {
    const int r = u / U8, c8 = u - r * U8;
    const int b = min(b0 + r, a.B - 1);
    const uint16_t* src = a.y + (size_t)b * a.T * D + c8 * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < a.T; ++t) {
      const uint4 q = ldg16(src + (size_t)t * D);
      const uint16_t* h = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += bf2f(h[e]);
    }
    uint4 w;
    w.x = pack_bf16x2(s[0] * inv_t, s[1] * inv_t);
    w.y = pack_bf16x2(s[2] * inv_t, s[3] * inv_t);
    w.z = pack_bf16x2(s[4] * inv_t, s[5] * inv_t);
    w.w = pack_bf16x2(s[6] * inv_t, s[7] * inv_t);
    *reinterpret_cast<uint4*>(&ps[r * PS + c8 * 8]) = w;
  }
  __syncthreads();

  // ---- S^T [HH x 64] = W1^T P^T; wave owns hidden blocks wave NH + j
  f32x16 acc[NH][2];
#pragma unroll
  for (int j = 0; j < NH; ++j) acc[j][0] = acc[j][1] = f32x16{};
  for (int kb = 0; kb < D / 16; ++kb) {
    uint4 pb[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      pb[rb] = *reinterpret_cast<const uint4*>(&ps[(rb * 32 + l32) * PS + kb * 16 + h32 * 8]);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const uint4 wf = ldg16(a.head_w1 + ((size_t)(wave * NH + j) * (D / 16) + kb) * FRAG_ELEMS + lane * 8);
      acc[j][0] = mfma32(wf, pb[0], acc[j][0]);
      acc[j][1] = mfma32(wf, pb[1], acc[j][1]);
    }
  }

  // ---- logit = rho(ReLU(S)) . w2: each lane sums its hidden units in a
  // fixed order, then the lane pair (l, l ^ 32), then the four waves
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int hid = (wave * NH + j) * 32 + 8 * (v / 4) + 4 * h32 + v % 4;
        const float hv = bf2f(f2bf(fmaxf(acc[j][rb][v], 0.f)));
        part[rb] += hv * bf2f(a.head_w2[hid]);
      }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    part[rb] += __shfl_xor(part[rb], 32, 64);
    if (h32 == 0) red[wave][rb * 32 + l32] = part[rb];
  }
  __syncthreads();
  if (tid < IO_BM && b0 + tid < a.B)
    a.logits[b0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

template <int NH>
hipError_t launch_tok_h(const IoArgs& a, int D, hipStream_t s) {
  const int grid = a.T * ((a.B + IO_BM - 1) / IO_BM);
  switch (D / 128) {
    case 1: hipLaunchKernelGGL((tok_kernel<NH, 1>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    case 2: hipLaunchKernelGGL((tok_kernel<NH, 2>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((tok_kernel<NH, 4>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    case 6: hipLaunchKernelGGL((tok_kernel<NH, 6>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ND>
hipError_t launch_head_d(const IoArgs& a, hipStream_t s) {
  const int grid = (a.B + IO_BM - 1) / IO_BM;
  switch (a.head_hidden / 128) {
    case 1: hipLaunchKernelGGL((head_kernel<ND, 1>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    case 2: hipLaunchKernelGGL((head_kernel<ND, 2>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((head_kernel<ND, 4>), dim3(grid), dim3(IO_NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool io_width_supported(int D) { return D == 128 || D == 256 || D == 512 || D == 768; }
bool io_tok_hidden_supported(int h) { return h == 128 || h == 256 || h == 512 || h == 768; }
bool io_head_hidden_supported(int h) { return h == 128 || h == 256 || h == 512; }

hipError_t launch_tokenize(const IoArgs& a, hipStream_t s) {
  switch (a.tok_hidden / 128) {
    case 1: return launch_tok_h<1>(a, a.D, s);
    case 2: return launch_tok_h<2>(a, a.D, s);
    case 4: return launch_tok_h<4>(a, a.D, s);
    case 6: return launch_tok_h<6>(a, a.D, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head(const IoArgs& a, hipStream_t s) {
  switch (a.D / 128) {
    case 1: return launch_head_d<1>(a, s);
    case 2: return launch_head_d<2>(a, s);
    case 4: return launch_head_d<4>(a, s);
    case 6: return launch_head_d<6>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tmx
