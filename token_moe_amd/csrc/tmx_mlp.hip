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
  static constexpr int DEPTH = (W <= 256) ? 8 : (W <= 512) ? 4 : 2;  // weight prefetch distance (steps)
  static constexpr int NBR = NBO > 2 ? NBO : 2;     // fragments per step
  static constexpr int YS = (S1 - S2) / 2;          // ping-pong barrier step inside GEMM1
  static_assert(W % 128 == 0, "W must be a multiple of 128");
  static_assert(S1 % DEPTH == 0 && S2 % DEPTH == 0 && DEPTH % 2 == 0,
                "ring slots must line up across phases and chunks");
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// silu(z) = z * sigmoid(z) with the hardware exp and reciprocal (~1 ulp
// each); the result is rounded to bf16 right after, so this is exact enough.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <int W, int MODE>
__global__ __launch_bounds__(NT, 1) void mlp_kernel(const MlpArgs a) {
  using S = MlpShape<W>;
  constexpr int BM = S::BM, XS = S::XS, US = S::US, RBW = S::RBW, NBO = S::NBO;
  constexpr int S1 = S::S1, S2 = S::S2, NS = S::S, DEPTH = S::DEPTH, NBR = S::NBR, HC = S::HC, YS = S::YS;
  constexpr int U8 = W / 8;                    // 16-byte units per row
  constexpr int NPRO = BM * U8 / NT;           // row units per lane per tile
  constexpr int NE = (BM / 2) * U8 / NT;       // per row half
  static_assert((BM * U8) % NT == 0 && ((BM / 2) * U8) % NT == 0, "row units must divide evenly");

  // LDS: x_hat tile + two U buffers during the main loop; between tiles the
  // same bytes hold the fp32 output tile (all rows at once when it fits in
  // 160 KB, else one row half at a time). Stage row stride W + 4 floats: 16
  // consecutive rows land on distinct 16-byte bank groups.
  constexpr int XBYTES = BM * XS * 2, UBYTES = 2 * BM * US * 2;
  constexpr int SS = W + 4;
  constexpr int ROWTAB = 4 * BM * 4;
  constexpr int NPART = (BM * SS * 4 + ROWTAB <= 160 * 1024) ? 1 : 2;
  constexpr int SBYTES = (BM / NPART) * SS * 4;
  constexpr int SMEM = (XBYTES + UBYTES > SBYTES) ? XBYTES + UBYTES : SBYTES;
  static_assert(SMEM + ROWTAB <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ int rowb[2][BM];
  __shared__ int rowent[2][BM];
  uint16_t* const xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const us = reinterpret_cast<uint16_t*>(smem + XBYTES);
  float* const stage = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps addresses scalar
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const int wr = wave >> 2;                 // row half
  const int wc = wave & 3;                  // column quarter
  const int row0 = wr * (BM / 2);

  // ---- tiles ------------------------------------------------------------------
  // The kernel is persistent: workgroup i walks tiles i, i + G, i + 2G, ...
  // (G = grid size, a multiple of 8 when there are more tiles than
  // workgroups). Tile index j sits on XCD j % 8 -- the XCD that dispatches
  // workgroup j % G -- and with P % 8 == 0 XCD x owns the contiguous
  // positions [x*P/8, (x+1)*P/8): a position's weights stay in that XCD's L2,
  // and neighbouring mixed positions, whose Mix segments share cache lines of
  // the block-layout rows, are read and written by the same XCD.
  // Position units: one position, or with `pair` two adjacent positions
  // whose Mix segments are adjacent in memory (p and p+1 of one token share
  // each 2*D/H-element run), so a tile's loads and stores cover whole runs
  // instead of every other half of them.
  const bool pair = (MODE != MLP_ROUTED) && a.pair;
  constexpr int HB = BM / 2;                 // rows of one position in a paired tile
  const int NPU = pair ? a.P / 2 : a.P;
  const int per_pos = (MODE == MLP_ROUTED) ? a.max_tiles : a.rtiles;
  const int total = NPU * per_pos;
  struct Tile {
    int p, t, group, start, nrows;
  };
  auto decode = [&](int j, Tile& T) -> bool {
    int pu;
    if ((NPU & 7) == 0) {
      const int xcd = j & 7, q = j >> 3;
      pu = xcd * (NPU >> 3) + q / per_pos;
      T.t = q % per_pos;
    } else {
      pu = j / per_pos;
      T.t = j % per_pos;
    }
    T.p = pair ? 2 * pu : pu;
    if (MODE == MLP_ROUTED) {
      if (T.t >= a.ntiles[T.p]) return false;
      const int4 tl = a.tiles[(size_t)T.p * a.max_tiles + T.t];
      T.group = T.p * a.E + tl.x;
      T.start = tl.y;
      T.nrows = tl.z;
    } else {
      const int rb = pair ? HB : BM;
      T.group = T.p;
      T.start = T.t * rb;
      T.nrows = min(rb, a.B - T.start);
    }
    return true;
  };
  // position of tile row r
  auto rowpos = [&](const Tile& T, int r) -> int { return T.p + ((pair && r >= HB) ? 1 : 0); };
  auto next_valid = [&](int j, Tile& T) -> int {
    while (j < total && !decode(j, T)) j += gridDim.x;
    return j;
  };
  auto set_rows = [&](const Tile& T, int buf) {
    for (int r = tid; r < BM; r += NT) {
      int b = -1, ent = 0;
      if (MODE == MLP_ROUTED) {
        if (r < T.nrows) {
          ent = a.rows[(size_t)T.p * a.B * a.top_k + T.start + r];
          b = ent / a.top_k;
        }
      } else {
        const int rr = (pair && r >= HB) ? r - HB : r;   // row within its position
        if (rr < T.nrows) b = T.start + rr;
      }
      rowb[buf][r] = b;
      rowent[buf][r] = ent;
    }
  };

  // ---- weight fragment stream -------------------------------------------------
  const int NC = a.hidden / HC;
  const int NBh = a.hidden / 32;            // hidden 32-blocks of the whole MLP
  const int KBd = a.hidden / 16;            // GEMM2 k-steps over the whole hidden
  struct Stream {
    const uint16_t* gu;
    const uint16_t* d;
    int rot;
  };
  // Hidden chunks are visited in a rotated order (chunk (c + t) mod NC at
  // iteration c, t = row tile): the sum over chunks is the same, and the
  // workgroups of one position, which run side by side on one XCD, stream
  // different parts of the weights.
  // (with `pair` the row group wr computes position p + wr and streams its weights)
  auto bind = [&](const Tile& T) -> Stream {
    const int g = T.group + (pair ? wr : 0);
    return Stream{a.wgu + (size_t)g * NBh * (W / 16) * 2 * FRAG_ELEMS,
                  a.wd + (size_t)g * KBd * (W / 32) * FRAG_ELEMS, T.t % NC};
  };
  uint4 ring[DEPTH][NBR];
  // step s of chunk c: GEMM1 k-step s (< S1): gate and up fragments of hidden
  // block 4c + wc; GEMM2 k-step s - S1: down fragments of this wave's columns
  auto issue = [&](uint4* dst, const Stream& w, int c, int s) {
    c += w.rot;
    if (c >= NC) c -= NC;
    if (s < S1) {
      const uint16_t* f = w.gu + ((size_t)((c * 4 + wc) * (W / 16) + s) * 2) * FRAG_ELEMS + lane * 8;
      dst[0] = ldg16(f);
      dst[1] = ldg16(f + FRAG_ELEMS);
    } else {
      const int kb = c * (HC / 16) + (s - S1);
#pragma unroll
      for (int j = 0; j < NBO; ++j)
        dst[j] = ldg16(w.d + ((size_t)kb * (W / 32) + wc * NBO + j) * FRAG_ELEMS + lane * 8);
    }
  };
  // refill a ring slot with the fragments of step s of chunk c; a step past
  // the chunk end belongs to chunk c+1, and past the last chunk to chunk 0
  // of the workgroup's next tile (or, after its last tile, to a chunk that
  // is re-read and never used). The stream never stops and the loads are
  // issued unconditionally, so the wait counters stay uniform: a conditional
  // load here makes the compiler drain the whole ring (vmcnt(0)) at every
  // chunk boundary.
  Stream cw, nw;
  auto refill = [&](uint4* dst, int c, int s) {
    if (s >= NS) {
      s -= NS;
      const bool last = c + 1 >= NC;
      Stream w;
      w.gu = last ? nw.gu : cw.gu;
      w.d = last ? nw.d : cw.d;
      w.rot = last ? nw.rot : cw.rot;
      issue(dst, w, last ? 0 : c + 1, s);
    } else {
      issue(dst, cw, c, s);
    }
  };

  // ---- row I/O ----------------------------------------------------------------
  // Unit u = (row, 8 columns) of the tile; lane-consecutive units cover one
  // row. Every global access of the rows is one 16-byte vector (8 columns
  // never straddle a Mix segment since D/H % 8 == 0).
  auto load_x = [&](int tix, int buf, const Tile& T, uint4* v) {
#pragma unroll
    for (int i = 0; i < NPRO; ++i) {
      const int u = tix + i * NT;
      const int r = u / U8, c8 = u - r * U8;
      const int b = rowb[buf][r];
      v[i] = make_uint4(0, 0, 0, 0);
      if (b >= 0) {
        const int p = rowpos(T, r);
        if (MODE == MLP_DENSE)
          v[i] = ldg16(a.x + a.map.offset(b, p, c8 * 8));
        else
          v[i] = ldg16(a.xhat + ((size_t)p * a.B + b) * W + c8 * 8);
      }
    }
  };
  // x rows -> LDS x_hat; for DENSE the RMS statistics reduce across the lanes
  // of a row before x_hat is written (RMSNorm in fp32, rho to bf16:
  // TokenMixer-Large section 2.3.3)
  auto store_x = [&](int tix, uint4* v) {
    constexpr bool kFusedNorm = (U8 <= 64 || U8 % 64 == 0);
    if constexpr (MODE == MLP_DENSE && kFusedNorm) {
      constexpr int LPR = U8 < 64 ? U8 : 64;  // lanes per row within a wave
      constexpr int WPR = U8 > 64 ? U8 / 64 : 1;
      float ss[NPRO];
#pragma unroll
      for (int i = 0; i < NPRO; ++i) {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[i]);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = bf2f(h[e]);
          acc += f * f;
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
        ss[i] = acc;
      }
      if (WPR > 1) {
        // rows wider than a wave: combine the per-wave partial sums in LDS
        float* red = reinterpret_cast<float*>(us);
#pragma unroll
        for (int i = 0; i < NPRO; ++i)
          if (lane == 0) red[i * (NT / 64) + wave] = ss[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NPRO; ++i) {
          const int w0 = (wave / WPR) * WPR;
          float t = 0.f;
          for (int w = 0; w < WPR; ++w) t += red[i * (NT / 64) + w0 + w];
          ss[i] = t;
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < NPRO; ++i) {
        const int u = tix + i * NT;
        const int c8 = u % U8;
        const float rinv = 1.0f / sqrtf(ss[i] / (float)W + a.eps);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[i]);
        float n[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) n[e] = bf2f(h[e]) * rinv * a.gain[c8 * 8 + e];
        v[i].x = pack_bf16x2(n[0], n[1]);
        v[i].y = pack_bf16x2(n[2], n[3]);
        v[i].z = pack_bf16x2(n[4], n[5]);
        v[i].w = pack_bf16x2(n[6], n[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < NPRO; ++i) {
      const int u = tix + i * NT;
      const int r = u / U8, c8 = u - r * U8;
      *reinterpret_cast<uint4*>(&xs[r * XS + c8 * 8]) = v[i];
    }
    __syncthreads();
    if constexpr (MODE == MLP_DENSE && !kFusedNorm) {
      // rows that do not tile waves: one wave per row, in place in LDS
      for (int r = wave; r < BM; r += NT / 64) {
        float acc = 0.f;
        for (int c8 = lane; c8 < U8; c8 += 64) {
          const uint4 q = *reinterpret_cast<const uint4*>(&xs[r * XS + c8 * 8]);
          const uint16_t* h = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = bf2f(h[e]);
            acc += f * f;
          }
        }
        acc = wave_sum(acc);
        const float rinv = 1.0f / sqrtf(acc / (float)W + a.eps);
        for (int c8 = lane; c8 < U8; c8 += 64) {
          uint4 q = *reinterpret_cast<const uint4*>(&xs[r * XS + c8 * 8]);
          const uint16_t* h = reinterpret_cast<const uint16_t*>(&q);
          float n[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) n[e] = bf2f(h[e]) * rinv * a.gain[c8 * 8 + e];
          q.x = pack_bf16x2(n[0], n[1]);
          q.y = pack_bf16x2(n[2], n[3]);
          q.z = pack_bf16x2(n[4], n[5]);
          q.w = pack_bf16x2(n[6], n[7]);
          *reinterpret_cast<uint4*>(&xs[r * XS + c8 * 8]) = q;
        }
      }
      __syncthreads();
    }
  };
  // residual rows of the tile, same unit order as load_x
  auto load_resid = [&](int tix, int buf, const Tile& T, uint4* rv) {
#pragma unroll
    for (int i = 0; i < NPRO; ++i) {
      const int u = tix + i * NT;
      const int r = u / U8, c8 = u - r * U8;
      const int b = rowb[buf][r];
      rv[i] = b >= 0 ? ldg16(a.resid + a.map.offset(b, rowpos(T, r), c8 * 8)) : make_uint4(0, 0, 0, 0);
    }
  };

  // ---- first tile ---------------------------------------------------------------
  Tile cur, nx;
  int ci = next_valid(blockIdx.x, cur);
  if (ci >= total) return;                                     // uniform per workgroup
  int ni = next_valid(ci + gridDim.x, nx);
  int buf = 0;
  set_rows(cur, 0);
  cw = bind(cur);
  nw = ni < total ? bind(nx) : cw;
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) issue(ring[s], cw, 0, s);
  __syncthreads();
  {
    uint4 v[NPRO];
    load_x(tid, 0, cur, v);
    store_x(tid, v);
  }

  while (true) {
    // ---- main loop ---------------------------------------------------------------
    f32x16 oacc[RBW][NBO];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int j = 0; j < NBO; ++j) oacc[i][j] = f32x16{};

    // Ping-pong of the two row groups (wr = 0: A, wr = 1: B). Each chunk is
    //   GEMM1 steps [0, YS) | barrier Y | GEMM1 steps [YS, S1) + U | barrier X | GEMM2
    // and group B runs one extra barrier before the loop, group A one after
    // it, so A's X pairs with B's Y and A's Y with B's X: while one group
    // computes silu(gate)*up on the VALU, the other group's waves on the same
    // SIMDs keep the MFMA pipe busy. Each group reads only its own U rows,
    // after its own X barrier; a U buffer is rewritten only after the next Y
    // barrier, which every wave reaches after finishing its GEMM2 reads.
    if (wr == 1) __syncthreads();

    for (int c = 0; c < NC; ++c) {
      uint16_t* ub = us + (c & 1) * BM * US;
      f32x16 sg[RBW], su[RBW];
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        sg[i] = f32x16{};
        su[i] = f32x16{};
      }

      // GEMM1 (fully unrolled: ring slots and the barrier point are
      // compile-time). The x_hat fragments of step s+1 are read from LDS while
      // step s runs; sched_barrier pins each step's loads where they are issued.
      uint4 xa[2][RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        xa[0][rb] = *reinterpret_cast<const uint4*>(&xs[(row0 + rb * 32 + l32) * XS + h32 * 8]);
#pragma unroll
      for (int s = 0; s < S1; ++s) {
        if (s == YS) __syncthreads();                              // barrier Y
        const int d = s % DEPTH;
        if (s + 1 < S1) {
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            xa[(s + 1) & 1][rb] =
                *reinterpret_cast<const uint4*>(&xs[(row0 + rb * 32 + l32) * XS + (s + 1) * 16 + h32 * 8]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          // S^T = W^T x_hat^T: the packed weight fragment is the A operand
          // (W^T rows = hidden units) and the x_hat rows are the B operand
          sg[rb] = mfma32(ring[d][0], xa[s & 1][rb], sg[rb]);
          su[rb] = mfma32(ring[d][1], xa[s & 1][rb], su[rb]);
        }
        refill(ring[d], c, s + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
      }

      // U = rho(silu(gate) * up). C layout of S^T (32 hidden x 32 rows): lane
      // holds row l32 and hidden 8*(v/4) + 4*h32 + v%4, i.e. 4 consecutive
      // hidden units per v-group -> one 8-byte LDS store each
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const int row = row0 + rb * 32 + l32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float uv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) uv[i] = silu_fast(sg[rb][4 * g4 + i]) * su[rb][4 * g4 + i];
          uint2 w2;
          w2.x = pack_bf16x2(uv[0], uv[1]);
          w2.y = pack_bf16x2(uv[2], uv[3]);
          *reinterpret_cast<uint2*>(&ub[row * US + wc * 32 + 8 * g4 + 4 * h32]) = w2;
        }
      }
      __syncthreads();                                             // barrier X

      // GEMM2: O^T += W_down[chunk]^T U^T, U fragments read one step ahead
      uint4 ua[2][RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        ua[0][rb] = *reinterpret_cast<const uint4*>(&ub[(row0 + rb * 32 + l32) * US + h32 * 8]);
#pragma unroll
      for (int k2 = 0; k2 < S2; ++k2) {
        const int d = (S1 + k2) % DEPTH;
        if (k2 + 1 < S2) {
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            ua[(k2 + 1) & 1][rb] =
                *reinterpret_cast<const uint4*>(&ub[(row0 + rb * 32 + l32) * US + (k2 + 1) * 16 + h32 * 8]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
          for (int j = 0; j < NBO; ++j) oacc[rb][j] = mfma32(ring[d][j], ua[k2 & 1][rb], oacc[rb][j]);   // O^T block
        refill(ring[d], c, S1 + k2 + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (wr == 0) __syncthreads();

    // ---- between tiles: stage O, start the next tile's loads, epilogue --------
    // The ring already holds the next tile's first fragments (see refill).
    const bool has_next = ni < total;
    if (has_next) set_rows(nx, buf ^ 1);
    // an opaque copy of the thread index: keeps the compiler from hoisting
    // the epilogue's and the next prologue's address arithmetic out of the
    // tile loop, where it would stay live through the main loop
    int etid = tid;
    asm volatile("" : "+v"(etid));
    constexpr bool PREF_R = (NPART == 1) && (MODE != MLP_ROUTED);
    constexpr int PR = BM / NPART;           // rows per staged part
    constexpr int NE = PR * U8 / NT;         // units per lane per part
    static_assert((PR * U8) % NT == 0, "part units must divide evenly");
    uint4 pr[PREF_R ? NPRO : 1];
    // defined on every path: a conditionally written px becomes a value
    // carried around the tile loop and stays live through the main loop
    uint4 px[NPRO];
#pragma unroll
    for (int i = 0; i < NPRO; ++i) px[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      __syncthreads();
      if (NPART == 1 || wr == part) {
        // C layout of an O^T block (32 columns x 32 rows): lane holds row l32
        // and columns 8*(v/4) + 4*h32 + v%4 -> 4 consecutive columns per v-group
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
          for (int j = 0; j < NBO; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int r = (NPART == 1 ? row0 : 0) + rb * 32 + l32;
              const int col = (wc * NBO + j) * 32 + 8 * g4 + 4 * h32;
              *reinterpret_cast<float4*>(&stage[r * SS + col]) =
                  make_float4(oacc[rb][j][4 * g4], oacc[rb][j][4 * g4 + 1], oacc[rb][j][4 * g4 + 2],
                              oacc[rb][j][4 * g4 + 3]);
            }
      }
      __syncthreads();
      if (part == NPART - 1) {
        if constexpr (PREF_R) load_resid(etid, buf, cur, pr);
        if (has_next) load_x(etid, buf ^ 1, nx, px);
      }
      // O goes out of LDS in 16-byte units: residual / extra / output through
      // the row map, partials as fp32 rows
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int u = etid + i * NT;
        const int r = u / U8, c8 = u - r * U8;
        const int R = part * PR + r;
        const int b = rowb[buf][R];
        if (b < 0) continue;
        const float4 o0 = *reinterpret_cast<const float4*>(&stage[r * SS + c8 * 8]);
        const float4 o1 = *reinterpret_cast<const float4*>(&stage[r * SS + c8 * 8 + 4]);
        float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        if (MODE == MLP_ROUTED) {
          const int slot = rowent[buf][R] - b * a.top_k;
          const size_t gi = ((size_t)b * a.P + cur.p) * a.top_k + slot;
          const float g = a.gate[gi];
          float4* dst = reinterpret_cast<float4*>(a.part + gi * W + c8 * 8);
          dst[0] = make_float4(g * o[0], g * o[1], g * o[2], g * o[3]);
          dst[1] = make_float4(g * o[4], g * o[5], g * o[6], g * o[7]);
        } else {
          const int p = rowpos(cur, R);
          if (MODE == MLP_SHARED) {
            const float* src = a.part + ((size_t)b * a.P + p) * a.top_k * W + c8 * 8;
            for (int sl = 0; sl < a.top_k; ++sl) {
              const float4 q0 = *reinterpret_cast<const float4*>(src + (size_t)sl * W);
              const float4 q1 = *reinterpret_cast<const float4*>(src + (size_t)sl * W + 4);
              o[0] += q0.x; o[1] += q0.y; o[2] += q0.z; o[3] += q0.w;
              o[4] += q1.x; o[5] += q1.y; o[6] += q1.z; o[7] += q1.w;
            }
          }
          const int64_t off = a.map.offset(b, p, c8 * 8);
          uint4 rvv;
          if constexpr (PREF_R) rvv = pr[i];
          else rvv = ldg16(a.resid + off);
          const uint16_t* rh = reinterpret_cast<const uint16_t*>(&rvv);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += bf2f(rh[e]);
          if (a.extra) {
            const uint4 ev = ldg16(a.extra + off);
            const uint16_t* eh = reinterpret_cast<const uint16_t*>(&ev);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += bf2f(eh[e]);
          }
          uint4 w;
          w.x = pack_bf16x2(o[0], o[1]);
          w.y = pack_bf16x2(o[2], o[3]);
          w.z = pack_bf16x2(o[4], o[5]);
          w.w = pack_bf16x2(o[6], o[7]);
          *reinterpret_cast<uint4*>(a.out + off) = w;
        }
      }
    }
    if (!has_next) break;
    __syncthreads();                       // staging reads done before x_hat is rewritten
    store_x(etid, px);
    cur = nx;
    ci = ni;
    buf ^= 1;
    cw = nw;
    ni = next_valid(ci + gridDim.x, nx);
    nw = ni < total ? bind(nx) : cw;
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

hipError_t launch_mlp(int mode, int W, const MlpArgs& a, int tiles, int workers, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  // persistent grid: at most `workers` workgroups, a multiple of 8 so that a
  // workgroup's tiles all sit on its own XCD
  workers &= ~7;
  const int grid = (workers <= 0 || tiles <= workers) ? tiles : workers;
  switch (W) {
    case 128: return launch_w<128>(mode, a, grid, s);
    case 256: return launch_w<256>(mode, a, grid, s);
    case 512: return launch_w<512>(mode, a, grid, s);
    case 768: return launch_w<768>(mode, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tmx
