// tmx_mlp.hip -- fused per-position SwiGLU MLP on gfx950 bf16 MFMA.
//
// One workgroup (4 waves, 256 lanes) owns BM rows of one position p (or of
// one (position, expert) bucket) and runs the whole pSwiGLU of TokenMixer-
// Large Eq. 17-18 on them without writing the hidden activations to HBM:
//
//   prologue  rows -> LDS tile  x_hat [BM, W] (bf16)
//             DENSE: rows are gathered through the Mix map (Eq. 9-11) and
//             RMS-normalised in LDS (section 2.3.3); ROUTED / SHARED read
//             the already normalised rows of the MoE path.
//   loop over hidden chunks of HC = 128:
//     GEMM1   S_gate, S_up [BM, HC] = x_hat @ W_gate/up[:, chunk]   (MFMA)
//     U       rho(silu(S_gate) * S_up) -> LDS (double buffered)
//     GEMM2   O [BM, W] += U @ W_down[chunk, :]                    (MFMA)
//   epilogue  DENSE : out = rho(resid + O [+ extra]) through the row map
//                    (for the mix sub-layer the store is the Revert map)
//             ROUTED: part[b, p, slot] = gate * O           (fp32)
//             SHARED: out = rho(resid + O + sum_slot part [+ extra])
//
// MFMA shape: v_mfma_f32_32x32x16_bf16 (measured on MI355X near the dense
// bf16 rate even at one wave per SIMD; the 16x16x32 form reaches about half).
// Wave roles: 8 waves (two per SIMD) as 2 (row halves) x 4 (columns). In
// GEMM1 wave (wr, wc) owns hidden units [32wc, 32wc+32) of the chunk for its
// BM/2 rows (a gate block and an up block, so silu(g)*u is lane-local); in
// GEMM2 it owns output columns [W/4 * wc, W/4 * (wc+1)) of its rows.
// x_hat and U fragments are read from LDS; weight fragments are pre-packed so
// a wave reads each one with a single 16-byte load per lane (each fragment is
// read by the two waves of a column).  The per-step weight fragments stream
// through a register ring that runs ahead across the GEMM1 / GEMM2 phases
// and across chunks.
#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int NT = 512;   // 8 waves

template <int W>
struct MlpShape {
  static constexpr int BM = (W <= 256) ? 128 : 64;  // rows per workgroup
  static constexpr int HC = MLP_HC;                 // hidden chunk
  static constexpr int XS = W + 8;                  // x_hat row stride (+16 B: rows on distinct banks)
  static constexpr int US = HC + 8;                 // U row stride
  static constexpr int RBW = BM / 64;               // 32-row blocks per wave (half the rows)
  static constexpr int NBO = W / 128;               // GEMM2 32-column blocks per wave
  static constexpr int S1 = W / 16;                 // GEMM1 k-steps per chunk
  static constexpr int S2 = HC / 16;                // GEMM2 k-steps per chunk
  static constexpr int S = S1 + S2;
  static constexpr int DEPTH = (W <= 512) ? 4 : 2;  // weight-fragment prefetch distance (steps)
  static constexpr int NBR = NBO > 2 ? NBO : 2;     // fragments per step
  static_assert(W % 128 == 0, "W must be a multiple of 128");
  static_assert(S1 % DEPTH == 0 && S2 % DEPTH == 0, "ring slots must line up across phases and chunks");
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <int W, int MODE>
__global__ __launch_bounds__(NT, 1) void mlp_kernel(const MlpArgs a) {
  using S = MlpShape<W>;
  constexpr int BM = S::BM, XS = S::XS, US = S::US, RBW = S::RBW, NBO = S::NBO;
  constexpr int S1 = S::S1, S2 = S::S2, NS = S::S, DEPTH = S::DEPTH, NBR = S::NBR, HC = S::HC;

  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * XS];
  __shared__ __attribute__((aligned(16))) uint16_t us[2 * BM * US];
  __shared__ int rowb[BM];
  __shared__ int rowent[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps addresses scalar
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const int wr = wave >> 2;                 // row half
  const int wc = wave & 3;                  // column quarter
  const int row0 = wr * (BM / 2);

  // ---- which tile: blocks of one position are kept on one XCD ------------
  // Workgroup i is dispatched to XCD i % 8; with P % 8 == 0 every XCD walks
  // the tiles of positions xcd, xcd + 8, ... so a position's weights stay in
  // that XCD's L2.
  const int per_pos = (MODE == MLP_ROUTED) ? a.max_tiles : a.rtiles;
  int p, t;
  {
    const int i = blockIdx.x;
    if ((a.P & 7) == 0) {
      const int xcd = i & 7, j = i >> 3;
      p = xcd + 8 * (j / per_pos);
      t = j % per_pos;
    } else {
      p = i / per_pos;
      t = i % per_pos;
    }
  }
  int group = p, nrows, start;
  if (MODE == MLP_ROUTED) {
    if (t >= a.ntiles[p]) return;                       // uniform per workgroup
    const int4 tl = a.tiles[(size_t)p * a.max_tiles + t];
    group = p * a.E + tl.x;
    start = tl.y;
    nrows = tl.z;
  } else {
    start = t * BM;
    nrows = min(BM, a.B - start);
  }

  for (int r = tid; r < BM; r += NT) {
    int b = -1, ent = 0;
    if (r < nrows) {
      if (MODE == MLP_ROUTED) {
        ent = a.rows[(size_t)p * a.B * a.top_k + start + r];
        b = ent / a.top_k;
      } else {
        b = start + r;
      }
    }
    rowb[r] = b;
    rowent[r] = ent;
  }

  // ---- weight fragment stream -------------------------------------------------
  const int NC = a.hidden / HC;
  const int NBh = a.hidden / 32;            // hidden 32-blocks of the whole MLP
  const int KBd = a.hidden / 16;            // GEMM2 k-steps over the whole hidden
  const uint16_t* wgu = a.wgu + (size_t)group * NBh * (W / 16) * 2 * FRAG_ELEMS;
  const uint16_t* wd = a.wd + (size_t)group * KBd * (W / 32) * FRAG_ELEMS;

  uint4 ring[DEPTH][NBR];
  // step s of chunk c: GEMM1 k-step s (< S1): gate and up fragments of hidden
  // block 4c + wc; GEMM2 k-step s - S1: down fragments of this wave's columns
  auto issue = [&](uint4* dst, int c, int s) {
    if (s < S1) {
      const uint16_t* f = wgu + ((size_t)((c * 4 + wc) * (W / 16) + s) * 2) * FRAG_ELEMS + lane * 8;
      dst[0] = ldg16(f);
      dst[1] = ldg16(f + FRAG_ELEMS);
    } else {
      const int kb = c * (HC / 16) + (s - S1);
#pragma unroll
      for (int j = 0; j < NBO; ++j)
        dst[j] = ldg16(wd + ((size_t)kb * (W / 32) + wc * NBO + j) * FRAG_ELEMS + lane * 8);
    }
  };
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) issue(ring[s], 0, s);

  __syncthreads();

  // ---- prologue: rows -> LDS ------------------------------------------------
  constexpr int U8 = W / 8;
  for (int u = tid; u < BM * U8; u += NT) {
    const int r = u / U8, c8 = u - r * U8;
    const int b = rowb[r];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (b >= 0) {
      if (MODE == MLP_DENSE)
        v = ldg16(a.x + a.map.offset(b, p, c8 * 8));
      else
        v = ldg16(a.xhat + ((size_t)p * a.B + b) * W + c8 * 8);
    }
    *reinterpret_cast<uint4*>(&xs[r * XS + c8 * 8]) = v;
  }
  __syncthreads();

  if (MODE == MLP_DENSE) {
    // RMSNorm per row (fp32 statistics), rho to bf16, in place.
    for (int r = wave; r < BM; r += NT / 64) {
      float ss = 0.f;
      for (int c8 = lane; c8 < U8; c8 += 64) {
        const uint4 v = *reinterpret_cast<const uint4*>(&xs[r * XS + c8 * 8]);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float f = bf2f(h[i]);
          ss += f * f;
        }
      }
      ss = wave_sum(ss);
      const float rinv = 1.0f / sqrtf(ss / (float)W + a.eps);
      for (int c8 = lane; c8 < U8; c8 += 64) {
        uint4 v = *reinterpret_cast<const uint4*>(&xs[r * XS + c8 * 8]);
        uint16_t* h = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = f2bf(bf2f(h[i]) * rinv * a.gain[c8 * 8 + i]);
        *reinterpret_cast<uint4*>(&xs[r * XS + c8 * 8]) = v;
      }
    }
    __syncthreads();
  }

  // ---- main loop ---------------------------------------------------------------
  f32x16 oacc[RBW][NBO];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int j = 0; j < NBO; ++j) oacc[i][j] = f32x16{};

  // refill a ring slot with the fragments of step s of chunk c (the step
  // index may run past the chunk into the next one)
  auto refill = [&](uint4* dst, int c, int s) {
    if (s < NS)
      issue(dst, c, s);
    else if (c + 1 < NC)
      issue(dst, c + 1, s - NS);
  };

  for (int c = 0; c < NC; ++c) {
    uint16_t* ub = us + (c & 1) * BM * US;
    f32x16 sg[RBW], su[RBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      sg[i] = f32x16{};
      su[i] = f32x16{};
    }

    // GEMM1: k-steps in groups of DEPTH so ring slots are compile-time
    for (int g = 0; g < S1 / DEPTH; ++g) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int s = g * DEPTH + d;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const uint4 af = *reinterpret_cast<const uint4*>(&xs[(row0 + rb * 32 + l32) * XS + s * 16 + h32 * 8]);
          sg[rb] = mfma32(af, ring[d][0], sg[rb]);
          su[rb] = mfma32(af, ring[d][1], su[rb]);
        }
        refill(ring[d], c, s + DEPTH);
      }
    }

    // U = rho(silu(gate) * up); C layout of 32x32: lane holds column l32,
    // rows 8*(v/4) + 4*h32 + v%4 of each 32-row block
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + rb * 32 + 8 * (v >> 2) + 4 * h32 + (v & 3);
        ub[row * US + wc * 32 + l32] = f2bf(silu(sg[rb][v]) * su[rb][v]);
      }
    __syncthreads();

    // GEMM2: O += U @ W_down[chunk]
#pragma unroll
    for (int g = 0; g < S2 / DEPTH; ++g) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int k2 = g * DEPTH + d;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const uint4 af = *reinterpret_cast<const uint4*>(&ub[(row0 + rb * 32 + l32) * US + k2 * 16 + h32 * 8]);
#pragma unroll
          for (int j = 0; j < NBO; ++j) oacc[rb][j] = mfma32(af, ring[d][j], oacc[rb][j]);
        }
        refill(ring[d], c, S1 + k2 + DEPTH);
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  // column part of the block-layout offset, once per output column block
  int64_t coloff[NBO];
#pragma unroll
  for (int j = 0; j < NBO; ++j) coloff[j] = a.map.offset(0, p, (wc * NBO + j) * 32 + l32);
  const int64_t rowstride = (int64_t)a.map.T * a.map.D;

#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = row0 + rb * 32 + 8 * (v >> 2) + 4 * h32 + (v & 3);
      const int b = rowb[r];
      if (b < 0) continue;
      if (MODE == MLP_ROUTED) {
        const int s = rowent[r] - b * a.top_k;
        const size_t gi = ((size_t)b * a.P + p) * a.top_k + s;
        const float g = a.gate[gi];
        float* dst = a.part + gi * W + wc * NBO * 32 + l32;
#pragma unroll
        for (int j = 0; j < NBO; ++j) dst[j * 32] = g * oacc[rb][j][v];
      } else {
        const int64_t rbase = (int64_t)b * rowstride;
#pragma unroll
        for (int j = 0; j < NBO; ++j) {
          const int64_t off = rbase + coloff[j];
          float val = oacc[rb][j][v];
          if (MODE == MLP_SHARED) {
            const float* src = a.part + ((size_t)b * a.P + p) * a.top_k * W + (wc * NBO + j) * 32 + l32;
            for (int s = 0; s < a.top_k; ++s) val += src[(size_t)s * W];
          }
          val += bf2f(a.resid[off]);
          if (a.extra) val += bf2f(a.extra[off]);
          a.out[off] = f2bf(val);
        }
      }
    }
}

template <int W>
hipError_t launch_w(int mode, const MlpArgs& a, int grid, hipStream_t s) {
  switch (mode) {
    case MLP_DENSE: hipLaunchKernelGGL((mlp_kernel<W, MLP_DENSE>), dim3(grid), dim3(NT), 0, s, a); break;
    case MLP_ROUTED: hipLaunchKernelGGL((mlp_kernel<W, MLP_ROUTED>), dim3(grid), dim3(NT), 0, s, a); break;
    default: hipLaunchKernelGGL((mlp_kernel<W, MLP_SHARED>), dim3(grid), dim3(NT), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool mlp_width_supported(int W) { return W == 128 || W == 256 || W == 512 || W == 768; }

int mlp_bm_for_width(int W) { return W <= 256 ? 128 : 64; }

hipError_t launch_mlp(int mode, int W, const MlpArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (W) {
    case 128: return launch_w<128>(mode, a, grid, s);
    case 256: return launch_w<256>(mode, a, grid, s);
    case 512: return launch_w<512>(mode, a, grid, s);
    case 768: return launch_w<768>(mode, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tmx
