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
//   loop over hidden chunks of HC = 64:
//     GEMM1   S_gate, S_up [BM, HC] = x_hat @ W_gate/up[:, chunk]   (MFMA)
//     U       rho(silu(S_gate) * S_up) -> LDS (double buffered)
//     GEMM2   O [BM, W] += U @ W_down[chunk, :]                    (MFMA)
//   epilogue  DENSE : out = rho(resid + O [+ extra]) through the row map
//                    (for the mix sub-layer the store is the Revert map)
//             ROUTED: part[b, p, slot] = gate * O           (fp32)
//             SHARED: out = rho(resid + O + sum_slot part [+ extra])
//
// Wave roles: GEMM1 splits the tile 2 (rows) x 2 (hidden) between the
// waves; GEMM2 splits the W output columns 4 ways.  x_hat and U fragments
// come from LDS; weight fragments are pre-packed so every lane issues one
// 16-byte global load per fragment and each fragment is read by at most two
// waves.  The O accumulator stays in registers for the whole K loop.
#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int NT = 256;
constexpr int HC = 64;          // hidden chunk
constexpr int US = HC + 8;      // U row stride (elements); +16 B keeps rows on distinct banks

template <int W>
struct MlpShape {
  static constexpr int BM = (W <= 256) ? 128 : 64;
  static constexpr int XS = W + 8;            // x_hat row stride (elements)
  static constexpr int KB1 = W / 32;          // GEMM1 k-steps
  static constexpr int RB1 = BM / 32;         // GEMM1 16-row blocks per wave
  static constexpr int RB2 = BM / 16;         // GEMM2 16-row blocks (all rows)
  static constexpr int NBW = W / 64;          // GEMM2 16-col blocks per wave
  static_assert(W % 64 == 0, "W must be a multiple of 64");
  static_assert(KB1 % 2 == 0, "double buffer assumes an even number of k-steps");
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int W, int MODE>
__global__ __launch_bounds__(NT, 1) void mlp_kernel(const MlpArgs a) {
  using S = MlpShape<W>;
  constexpr int BM = S::BM, XS = S::XS, KB1 = S::KB1, RB1 = S::RB1, RB2 = S::RB2, NBW = S::NBW;

  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * XS];
  __shared__ __attribute__((aligned(16))) uint16_t us[2 * BM * US];
  __shared__ int rowb[BM];
  __shared__ int rowent[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int q = lane >> 4;

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
  const int NC = a.hidden / HC;
  const int NBh = a.hidden / 16;            // hidden 16-blocks of the whole MLP
  const int KB2 = a.hidden / 32;            // GEMM2 k-steps over the whole hidden
  const uint16_t* wgu = a.wgu + (size_t)group * NBh * KB1 * 2 * FRAG_ELEMS;
  const uint16_t* wd = a.wd + (size_t)group * KB2 * (W / 16) * FRAG_ELEMS;
  const int wr = wave >> 1, wc = wave & 1;  // GEMM1 role

  f32x4 oacc[RB2][NBW];
#pragma unroll
  for (int i = 0; i < RB2; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // GEMM1 B fragments: [buf][nb2*2 + which]
  uint4 b1[2][4];
  uint4 b2[2][NBW];

  auto load_b1 = [&](uint4* dst, int c, int kb) {
#pragma unroll
    for (int nb2 = 0; nb2 < 2; ++nb2) {
      const int hb = c * 4 + wc * 2 + nb2;
      const uint16_t* f = wgu + ((size_t)(hb * KB1 + kb) * 2) * FRAG_ELEMS + lane * 8;
      dst[nb2 * 2 + 0] = ldg16(f);
      dst[nb2 * 2 + 1] = ldg16(f + FRAG_ELEMS);
    }
  };
  auto load_b2 = [&](int c) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int kb = c * 2 + kb2;
        const int nb = wave * NBW + j;
        b2[kb2][j] = ldg16(wd + ((size_t)kb * (W / 16) + nb) * FRAG_ELEMS + lane * 8);
      }
  };

  load_b1(b1[0], 0, 0);
  for (int c = 0; c < NC; ++c) {
    uint16_t* ub = us + (c & 1) * BM * US;
    f32x4 sg[RB1][2], su[RB1][2];
#pragma unroll
    for (int i = 0; i < RB1; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        su[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

#pragma unroll
    for (int kb = 0; kb < KB1; ++kb) {
      if (kb + 1 < KB1)
        load_b1(b1[(kb + 1) & 1], c, kb + 1);
      else
        load_b2(c);
      const uint4* bb = b1[kb & 1];
#pragma unroll
      for (int rb = 0; rb < RB1; ++rb) {
        const int row = wr * (BM / 2) + rb * 16 + l16;
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(&xs[row * XS + kb * 32 + q * 8]));
#pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2) {
          sg[rb][nb2] = mfma16x16x32(af, as_bf16x8(bb[nb2 * 2 + 0]), sg[rb][nb2]);
          su[rb][nb2] = mfma16x16x32(af, as_bf16x8(bb[nb2 * 2 + 1]), su[rb][nb2]);
        }
      }
    }

    // U = rho(silu(gate) * up) into LDS; C layout: lane holds rows 4q+v, col l16
#pragma unroll
    for (int rb = 0; rb < RB1; ++rb)
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wr * (BM / 2) + rb * 16 + q * 4 + v;
          const int col = (wc * 2 + nb2) * 16 + l16;
          ub[row * US + col] = f2bf(silu(sg[rb][nb2][v]) * su[rb][nb2][v]);
        }
    __syncthreads();

    if (c + 1 < NC) load_b1(b1[0], c + 1, 0);

#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int rb = 0; rb < RB2; ++rb) {
        const int row = rb * 16 + l16;
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(&ub[row * US + kb2 * 32 + q * 8]));
#pragma unroll
        for (int j = 0; j < NBW; ++j) oacc[rb][j] = mfma16x16x32(af, as_bf16x8(b2[kb2][j]), oacc[rb][j]);
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------
#pragma unroll
  for (int rb = 0; rb < RB2; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = rb * 16 + q * 4 + v;
      const int b = rowb[r];
      if (b < 0) continue;
      if (MODE == MLP_ROUTED) {
        const int ent = rowent[r];
        const int s = ent - b * a.top_k;
        const size_t gi = ((size_t)b * a.P + p) * a.top_k + s;
        const float g = a.gate[gi];
        float* dst = a.part + gi * W;
#pragma unroll
        for (int j = 0; j < NBW; ++j) dst[(wave * NBW + j) * 16 + l16] = g * oacc[rb][j][v];
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const int col = (wave * NBW + j) * 16 + l16;
          const int64_t off = a.map.offset(b, p, col);
          float val = oacc[rb][j][v];
          if (MODE == MLP_SHARED) {
            const float* src = a.part + ((size_t)b * a.P + p) * a.top_k * W + col;
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
