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
#include <type_traits>

#include "tmx_internal.h"

namespace tmx {

namespace {

// Waves per workgroup for a row width. 8 waves (two per SIMD, two row
// groups, 256 registers each) hide one group's SiLU and row I/O behind the
// other group's MFMAs, and let a Mix tile hold two adjacent positions; they
// are used where a wave's 64 rows keep each weight fragment busy for two
// MFMAs (W = 256). 4 waves (one per SIMD, 512 registers each, every wave on
// all BM rows) double the reuse of each weight fragment where BM is only 64
// (W = 512 and 768: at W = 768 the 64 x 768 fp32 output tile fills the 256
// accumulator registers of each wave) and serve W = 128.
constexpr int mlp_waves(int W) { return W == 256 ? 8 : 4; }

// Workgroups per CU. The dense W = 256 sub-layer runs as two 4-wave
// workgroups of 64 rows per CU (256 registers per wave, as in the 8-wave
// tile) that start half a tile apart: while one streams its rows in and
// out, the other's MFMAs keep the SIMDs busy. In a single 8-wave workgroup
// both row groups cross every tile boundary together, so every CU moved its
// rows at the same moment while no MFMA ran.
constexpr int mlp_occupancy(int mode, int W) { return (mode == MLP_DENSE && W == 256) ? 2 : 1; }
constexpr int mlp_waves(int mode, int W) { return mlp_occupancy(mode, W) == 2 ? 4 : mlp_waves(W); }

template <int W, int NW, int OCC>
struct MlpShape {
  static constexpr int NT = 64 * NW;
  static constexpr int BM = (W <= 256 && OCC == 1) ? 128 : 64;  // rows per workgroup
  static constexpr int HC = MLP_HC;                 // hidden chunk
  static constexpr int XS = W + 8;                  // x_hat row stride (+16 B: rows on distinct banks)
  static constexpr int US = HC + 8;                 // U row stride
  static constexpr int NRG = NW / 4;                // row groups of waves
  static constexpr int RBW = BM / (32 * NRG);       // 32-row blocks per wave
  static constexpr int NBO = W / 128;               // GEMM2 32-column blocks per wave
  static constexpr int S1 = W / 16;                 // GEMM1 k-steps per chunk
  static constexpr int S2 = HC / 16;                // GEMM2 k-steps per chunk
  static constexpr int S = S1 + S2;
  static constexpr int DEPTH = (NW == 4) ? (W <= 512 ? 4 : 2) : (W <= 256) ? 8 : (W <= 512) ? 4 : 2;  // weight prefetch distance (steps)
  static constexpr int NBR = NBO > 2 ? NBO : 2;     // fragments per step
  static constexpr int YS = (S1 - S2) / 2;          // ping-pong barrier step inside GEMM1
  static_assert(W % 128 == 0, "W must be a multiple of 128");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(S1 % DEPTH == 0 && S2 % DEPTH == 0 && DEPTH % 2 == 0,
                "ring slots must line up across phases and chunks");
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Streaming (non-temporal) 16-byte accesses for the MoE row streams that are
// touched once per launch -- normalised rows, gated expert outputs, combined
// outputs -- so that they do not push the weight fragments, which every tile
// of a position or bucket re-reads, out of L2.
typedef unsigned int nt_v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  const nt_v4u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stg16_nt(void* p, const uint4 v) {
  nt_v4u w;
  w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
  __builtin_nontemporal_store(w, reinterpret_cast<nt_v4u*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 E4M3 x E4M3 -> fp32 with E8M0 block scales: lane l supplies the
// scale of (row l % 32, K-block l / 32) of its operand in byte OA of sa (A)
// and byte OB of sb (B). A lane's 32 operand bytes: 0-15 are K 16 (l / 32)
// + j of K-block 0, 16-31 the same of K-block 1.
__device__ __forceinline__ i32x8 join8(const uint4& a, const uint4& b) {
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
template <int OA, int OB>
__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, (int)sa, OB, (int)sb);
}
// scale-byte selectors from loop indices that are constants after unrolling
__device__ __forceinline__ f32x16 mfma8s(int oa, int ob, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb,
                                         const f32x16& c) {
  switch (oa * 4 + ob) {
    case 0: return mfma8<0, 0>(a, b, sa, sb, c);
    case 1: return mfma8<0, 1>(a, b, sa, sb, c);
    case 2: return mfma8<0, 2>(a, b, sa, sb, c);
    case 3: return mfma8<0, 3>(a, b, sa, sb, c);
    case 4: return mfma8<1, 0>(a, b, sa, sb, c);
    case 5: return mfma8<1, 1>(a, b, sa, sb, c);
    case 6: return mfma8<1, 2>(a, b, sa, sb, c);
    case 7: return mfma8<1, 3>(a, b, sa, sb, c);
    case 8: return mfma8<2, 0>(a, b, sa, sb, c);
    case 9: return mfma8<2, 1>(a, b, sa, sb, c);
    case 10: return mfma8<2, 2>(a, b, sa, sb, c);
    case 11: return mfma8<2, 3>(a, b, sa, sb, c);
    case 12: return mfma8<3, 0>(a, b, sa, sb, c);
    case 13: return mfma8<3, 1>(a, b, sa, sb, c);
    case 14: return mfma8<3, 2>(a, b, sa, sb, c);
    default: return mfma8<3, 3>(a, b, sa, sb, c);
  }
}

// E4M3 bytes of x[0..3] * 2^-k (exact scaling), clamped to +-448 first: the
// hardware conversion rounds to nearest even but does not saturate
__device__ __forceinline__ uint32_t e4m3x4(float x0, float x1, float x2, float x3, float sc) {
  x0 = fminf(fmaxf(x0 * sc, -448.f), 448.f);
  x1 = fminf(fmaxf(x1 * sc, -448.f), 448.f);
  x2 = fminf(fmaxf(x2 * sc, -448.f), 448.f);
  x3 = fminf(fmaxf(x3 * sc, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}
// MX shared exponent of a block with largest magnitude amax: floor(log2(amax))
// - 8 (E4M3's largest normal is 1.75 * 2^8), clamped to the E8M0 range
__device__ __forceinline__ int mx_exp(float amax) {
  int e = 0;
  (void)frexpf(amax, &e);
  int k = amax > 0.f ? e - 9 : -127;
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// silu(z) = z * sigmoid(z) with the hardware exp and reciprocal (~1 ulp
// each); the result is rounded to bf16 right after, so this is exact enough.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Row variants of the epilogue (RV), one instantiation each, so that no
// epilogue load sits on one path only (the compiler would then wait for
// every load in flight, the next tile's rows and weights included):
//   RV_PLAIN   residual rows loaded, no inter-residual
//   RV_EXTRA   residual and inter-residual rows loaded (rows past the tile
//              end read row 0 and are not used)
//   RV_MIX     dense Mix sub-layer: the residual is the tile's own input
//              rows, read through the same map, so the raw rows stay in
//              registers from their load to the epilogue instead of being
//              read again (each Mix unit is a separate 2*D/H-byte run of a
//              token: those reads touch a cache line per run)
enum { RV_PLAIN = 0, RV_EXTRA = 1, RV_MIX = 2 };

// F8: the 4-wave kernels with MXFP8 GEMM operands -- dense W = 256 (two
// workgroups per CU), every mode at W = 512, the MoE modes at W = 768 (one)
// -- weights packed at load
// (launch_pack_mx), U and the DENSE rows quantised here per row and
// 32-element block along each GEMM's contraction axis; the MoE modes read
// the router's MXFP8 copy of x_hat (MlpArgs::xq8, xe8).
template <int W, int MODE, int NW, int OCC, int RV, bool F8>
__global__ __launch_bounds__(64 * NW, OCC) void mlp_kernel(const MlpArgs a) {
  constexpr bool RESX = RV == RV_MIX, EXTRA = RV == RV_EXTRA;
  static_assert(!F8 || (NW == 4 && ((W == 256 && MODE == MLP_DENSE && OCC == 2) || (W == 512 && OCC == 1) ||
                                    (W == 768 && MODE != MLP_DENSE && OCC == 1))),
                "MXFP8 kernel shape");
  static_assert(!RESX || MODE == MLP_DENSE, "input rows double as the residual only in dense sub-layers");
  static_assert(!EXTRA || MODE != MLP_ROUTED, "routed tiles have no residual");
  using S = MlpShape<W, NW, OCC>;
  constexpr int NT = S::NT;
  constexpr int BM = S::BM, XS = S::XS, US = S::US, RBW = S::RBW, NBO = S::NBO;
  constexpr int S1 = S::S1, S2 = S::S2, NS = S::S, DEPTH = S::DEPTH, NBR = S::NBR, HC = S::HC, YS = S::YS;
  constexpr int U8 = W / 8;                    // 16-byte units per row
  constexpr int NPRO = BM * U8 / NT;           // row units per lane per tile
  static_assert((BM * U8) % NT == 0, "row units must divide evenly");

  // LDS: x_hat tile + two U buffers during the main loop; between tiles the
  // same bytes hold the fp32 output tile (all rows at once when it fits in
  // 160 KB, else one row half at a time). Stage row stride W + 4 floats: 16
  // consecutive rows land on distinct 16-byte bank groups.
  // F8 layout of the same bytes during the main loop: x_hat codes [BM][XSB],
  // two U code buffers [BM][USB], x_hat scale words [BM][2 DWX] (word 2 (s /
  // 4) + h, byte s % 4: 32-column block 2s + h, s = 64-column K-step), two U
  // scale-word buffers [BM][2] (word h, byte t: hidden block 2t + h of the
  // chunk), and at W = 256 the tile's weight scale records [4 waves][RECX /
  // 4][64][4 dwords]. From W = 512 the weight scales go to registers
  // instead, straight from global memory one chunk ahead of their use
  // (REC_REG): copying records into LDS takes the LDS DMA, after which the
  // compiler makes every LDS read wait for all loads in flight, the weight
  // stream included. The F8 kernels never use the bf16 layout.
  constexpr int XBYTES = BM * XS * 2, UBYTES = 2 * BM * US * 2;
  constexpr int SS = W + 4;
  constexpr int ROWTAB = 6 * BM * 4;
  constexpr bool REC_REG = F8 && W >= 512;
  constexpr int NPART = (BM * SS * 4 + ROWTAB <= 160 * 1024) ? 1 : 2;
  constexpr int SBYTES = (BM / NPART) * SS * 4;
  constexpr int XSB = W + 16, USB = HC + 16;
  constexpr int DWX = W / 256;                   // scale dwords per matrix, chunk and lane
  constexpr int XSCB = W / 32;                   // x_hat scale bytes per row
  constexpr int RECX = (3 * DWX * mx_max_chunks(W) + 3) & ~3;  // record dwords the LDS holds per lane
  // TP (MoE modes from W = 512): two phases per tile instead of the chunk
  // pipeline -- GEMM1 and U of every hidden chunk first, U of the whole
  // hidden kept in LDS (codes [BM][USBA], scales [BM][USCB] laid out like
  // x_hat's), then one GEMM2 over the whole hidden -- so the gate / up
  // accumulators and the output accumulators (4 or 6 column blocks per
  // wave) are never live together. (At W = 768 the pipeline spilled ~280
  // VGPRs; at W = 512 the routed kernel ran 16% slower with it. The dense
  // W = 512 kernel keeps the pipeline, which overlaps U with GEMM2.)
  constexpr bool TP = F8 && (W == 768 || (W == 512 && MODE != MLP_DENSE));
  constexpr int HMAX = mx_max_chunks(W) * HC;
  constexpr int USBA = HMAX + 16, USCB = HMAX / 32;
  constexpr int OFF_XSC = BM * XSB + (TP ? BM * USBA : 2 * BM * USB);
  constexpr int OFF_USC = OFF_XSC + BM * XSCB;
  constexpr int F8CODES = OFF_USC + (TP ? BM * USCB : 2 * BM * 8);
  constexpr int F8BYTES = F8CODES + (REC_REG ? 0 : 4 * RECX * 64 * 4);
  constexpr int SMEM0 = (XBYTES + UBYTES > SBYTES) ? XBYTES + UBYTES : SBYTES;
  constexpr int SMEM = F8 ? (F8BYTES > SBYTES ? F8BYTES : SBYTES) : SMEM0;
  static_assert(SMEM + ROWTAB <= 160 * 1024, "LDS budget");
  static_assert(NW == 8 || NPART == 1 || RBW == NPART, "4 waves stage one row block per part");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ int rowb[2][BM];
  __shared__ int rowgi[2][BM];       // ROUTED: flat (b, p, slot) index of the row
  __shared__ float rowg[2][BM];      // ROUTED: gate of the row
  uint16_t* const xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const us = reinterpret_cast<uint16_t*>(smem + XBYTES);
  float* const stage = reinterpret_cast<float*>(smem);
  uint8_t* const xs8 = smem;
  uint8_t* const us8 = smem + BM * XSB;
  uint8_t* const xsc8 = smem + OFF_XSC;
  uint8_t* const usc8 = smem + OFF_USC;
  uint32_t* const wsc8 = reinterpret_cast<uint32_t*>(smem + F8CODES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps addresses scalar
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const int wr = NW == 8 ? wave >> 2 : 0;   // row group
  const int wc = wave & 3;                  // column quarter
  const int row0 = wr * (BM / 2);

  // ---- per-lane columns -------------------------------------------------------
  // Row I/O moves 16-byte units (8 columns); unit u of a tile is row u / U8,
  // columns 8 * (u % U8). When NT is a multiple of U8 a lane's columns are
  // the same for every unit and tile, so the column part of the block-layout
  // offset (a division by D/H for the Mix map) and the RMSNorm gains are
  // computed once here.
  constexpr bool LANE_COL = (NT % U8) == 0;
  const int lw0 = (tid % U8) * 8;
  const int lcol = a.map.col(lw0);
  auto uoff = [&](int b, int p, int c8) -> int64_t {
    if constexpr (LANE_COL)
      return a.map.row(b) + a.map.pos(p) + lcol;
    else
      return a.map.offset(b, p, c8 * 8);
  };
  // the lane's 8 gains, loaded next to each tile's x rows (registers held
  // through the main loop would cost spills)
  auto load_gain = [&](float* g) {
    if constexpr (MODE == MLP_DENSE && LANE_COL) {
      const float4 g0 = *reinterpret_cast<const float4*>(a.gain + lw0);
      const float4 g1 = *reinterpret_cast<const float4*>(a.gain + lw0 + 4);
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
      g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    }
  };

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
  const bool pair = (NW == 8) && (MODE != MLP_ROUTED) && a.pair;
  constexpr int HB = BM / 2;                 // rows of one position in a paired tile
  const int NPU = pair ? a.P / 2 : a.P;
  const int per_pos = (MODE == MLP_ROUTED) ? a.max_tiles : a.rtiles;
  const int total = NPU * per_pos;
  struct Tile {
    int p, t, group, start, nrows;
  };
  auto decode = [&](int j, Tile& T) -> bool {
    int pu;
    // SHARED walks each XCD's positions from the last: the routed launch
    // before it wrote its expert outputs in ascending position order, so
    // the most recently written -- the ones most likely still in the
    // last-level cache -- are combined first
    const bool split = (NPU & 7) == 0;
    const int q = split ? j >> 3 : j;          // tile index within the XCD's range
    const int npx = split ? NPU >> 3 : NPU;    // positions in that range
    int k;
    if (MODE != MLP_ROUTED && a.ileave) {
      // positions 2m and 2m+1 alternate: row tile t of 2m, of 2m+1, t+1 of 2m, ...
      const int m = q / (2 * per_pos), r = q - m * 2 * per_pos;
      k = 2 * m + (r & 1);
      T.t = r >> 1;
    } else {
      k = q / per_pos;
      T.t = q % per_pos;
    }
    pu = (split ? (j & 7) * npx : 0) + (MODE == MLP_SHARED ? npx - 1 - k : k);
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
  // ROUTED tiles come from queues instead: bucket sizes are uneven, so a
  // fixed assignment would leave some workgroups with twice the work. With
  // P % 8 == 0 each XCD has a queue over its own positions (the position
  // ranges of the static mapping), else one queue covers all positions.
  // Entry k of a queue is the k-th non-empty tile of its positions in order;
  // heads are zeroed by the bucket kernel, which runs just before.
  __shared__ int qslot;
  const bool split_q = (a.P & 7) == 0;
  const int qx = split_q ? (int)(blockIdx.x & 7) : 0;
  const int NPX = split_q ? (a.P >> 3) : a.P;
  auto qdecode = [&](int k, Tile& T) -> bool {
    int p = qx * NPX;
    for (int q = 0; q < NPX; ++q, ++p) {
      const int n = a.ntiles[p];
      if (k < n) {
        const int4 tl = a.tiles[(size_t)p * a.max_tiles + k];
        T.p = p;
        T.t = k;
        T.group = p * a.E + tl.x;
        T.start = tl.y;
        T.nrows = tl.z;
        return true;
      }
      k -= n;
    }
    return false;
  };
  auto set_rows = [&](const Tile& T, int buf) {
    for (int r = tid; r < BM; r += NT) {
      int b = -1;
      if (MODE == MLP_ROUTED) {
        int gi = 0;
        float g = 0.f;
        if (r < T.nrows) {
          const int ent = a.rows[(size_t)T.p * a.B * a.top_k + T.start + r];   // b * top_k + slot
          b = ent / a.top_k;
          gi = (b * a.P + T.p) * a.top_k + (ent - b * a.top_k);
          g = a.gate[gi];
        }
        rowgi[buf][r] = gi;
        rowg[buf][r] = g;
      } else {
        const int rr = (pair && r >= HB) ? r - HB : r;   // row within its position
        if (rr < T.nrows) b = T.start + rr;
      }
      rowb[buf][r] = b;
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
    if constexpr (F8)   // one byte per weight: 2 W h gate/up bytes, W h down bytes per position
      return Stream{reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.wgu) +
                                                      (size_t)g * 2 * W * a.hidden),
                    reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.wd) +
                                                      (size_t)g * W * a.hidden),
                    T.t % NC};
    return Stream{a.wgu + (size_t)g * NBh * (W / 16) * 2 * FRAG_ELEMS,
                  a.wd + (size_t)g * KBd * (W / 32) * FRAG_ELEMS, T.t % NC};
  };
  uint4 ring[DEPTH][NBR];
  // step s of chunk c: GEMM1 k-step s (< S1): gate and up fragments of hidden
  // block 4c + wc; GEMM2 k-step s - S1: down fragments of this wave's columns
  auto issue = [&](uint4* dst, const Stream& w, int c, int s) __attribute__((always_inline)) {
    c += w.rot;
    if (c >= NC) c -= NC;
    if (s < S1) {
      const uint16_t* f = w.gu + ((size_t)((c * 4 + wc) * (W / 16) + s) * 2) * FRAG_ELEMS + lane * 8;
      dst[0] = ldg16(f);
      dst[1] = ldg16(f + FRAG_ELEMS);
      // whole-slot writes on every path keep the ring in registers (a slot
      // written in part on some paths is left in scratch memory)
#pragma unroll
      for (int j = 2; j < NBR; ++j) dst[j] = make_uint4(0, 0, 0, 0);
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

  // 4-wave tiles treat the ring as NFR single fragments in stream order:
  // fragment k of the stream sits in slot k % NFR. A GEMM1 step consumes
  // 2 fragments and a GEMM2 step NBO, so GEMM1 looks NFR / 2 steps ahead
  // instead of DEPTH (a weight stream that starts cold -- a new expert --
  // needs the longer look-ahead). f1 = fragment f of chunk c in that order:
  // GEMM1 step f / 2 (gate, up), then GEMM2 step (f - F1) / NBO.
  constexpr int NFR = DEPTH * NBR;
  // F8: the ring holds NFR8 whole 32-byte fragments (two 1 KiB halves each);
  // a GEMM1 step (64 K) takes gate and up, a GEMM2 step NBO fragments, all
  // of which must be in the ring at once
  constexpr int KS8 = W / 64, TS8 = HC / 64, NFR8 = NBO > 4 ? NBO : 4;
  constexpr int F1 = F8 ? 2 * KS8 : 2 * S1, F2 = F8 ? NBO * TS8 : NBO * S2, FS = F1 + F2;
  constexpr int NFRX = F8 ? NFR8 : NFR;
  static_assert(NW == 8 || (F1 % NFRX == 0 && F2 % NFRX == 0),
                "every GEMM phase must start on a ring boundary");
  static_assert(!F8 || (NFR8 <= F1 && NFR8 <= F2), "the look-ahead stays within the next GEMM phase");
  static_assert(!F8 || (NFR8 >= NBO && NFR8 >= 2), "a GEMM step's fragments fit in the ring together");
  i32x8 ring8[F8 ? NFR8 : 1];
  auto fslot = [&](int k) __attribute__((always_inline)) -> uint4& {
    return ring[(k % NFR) / NBR][(k % NFR) % NBR];
  };
  auto issue_frag = [&](uint4& dst, const Stream& w, int c, int f) __attribute__((always_inline)) {
    c += w.rot;
    if (c >= NC) c -= NC;
    if (f < F1) {
      dst = ldg16(w.gu + ((size_t)((c * 4 + wc) * (W / 16) + f / 2) * 2 + (f & 1)) * FRAG_ELEMS + lane * 8);
    } else {
      const int kb = c * (HC / 16) + (f - F1) / NBO;
      dst = ldg16(w.d + ((size_t)kb * (W / 32) + wc * NBO + (f - F1) % NBO) * FRAG_ELEMS + lane * 8);
    }
  };

  // F8 fragment f of chunk c: GEMM1 step f / 2, gate (f even) or up, of
  // hidden block 4c + wc; then GEMM2 step t = (f - F1) / NBO, column block
  // wc NBO + (f - F1) % NBO. Both 1 KiB halves in one call.
  auto issue_frag8 = [&](i32x8& dst, const Stream& w, int c, int f) __attribute__((always_inline)) {
    c += w.rot;
    if (c >= NC) c -= NC;
    const uint8_t* base;
    if (f < F1) {
      base = reinterpret_cast<const uint8_t*>(w.gu) + (((size_t)(c * 4 + wc) * KS8 + (f >> 1)) * 2 + (f & 1)) * 2048;
    } else {
      const int g = f - F1;
      base = reinterpret_cast<const uint8_t*>(w.d) + ((size_t)(c * TS8 + g / NBO) * (W / 32) + wc * NBO + g % NBO) * 2048;
    }
    dst = join8(*reinterpret_cast<const uint4*>(base + lane * 16), *reinterpret_cast<const uint4*>(base + 1024 + lane * 16));
  };

  // ---- row I/O ----------------------------------------------------------------
  // Unit u = (row, 8 columns) of the tile; lane-consecutive units cover one
  // row. Every global access of the rows is one 16-byte vector (8 columns
  // never straddle a Mix segment since D/H % 8 == 0).
  // unit i of lane tix: row r and 8-column group c8. With LANE_COL a lane's
  // column group is the same for every unit and its rows step by NT / U8,
  // so both come from tix once instead of per unit.
  auto unit_rc = [&](int tix, int i, int& r, int& c8) __attribute__((always_inline)) {
    if constexpr (LANE_COL) {
      r = tix / U8 + i * (NT / U8);
      c8 = tix % U8;
    } else {
      const int u = tix + i * NT;
      r = u / U8;
      c8 = u - r * U8;
    }
  };
  // Row loads are issued without branches, IOB units at a time: the lane
  // reads the batch's row indices first and rows past the tile end load row
  // 0, so the batch's loads go out back to back. With one batch (up to 16
  // units per lane) the padding rows are cleared after it. With several
  // (W = 768: 24 units, batches of 8 -- all index copies at once would spill
  // in the main loop) they are not: clearing a load's destination makes the
  // wave wait for that load, which would serialise the batches, and an
  // output row depends only on its own input row while no epilogue stores
  // or reads a padding row.
  constexpr int IOB = NPRO <= 16 ? NPRO : 8;
  static_assert(NPRO % IOB == 0, "row-load batches must divide the units per lane");
  auto load_x = [&](int tix, int buf, const Tile& T, uint4* v) {
#pragma unroll
    for (int i0 = 0; i0 < NPRO; i0 += IOB) {
      int bb[IOB];
#pragma unroll
      for (int k = 0; k < IOB; ++k) {
        int r, c8;
        unit_rc(tix, i0 + k, r, c8);
        bb[k] = rowb[buf][r];
      }
#pragma unroll
      for (int k = 0; k < IOB; ++k) {
        int r, c8;
        unit_rc(tix, i0 + k, r, c8);
        const int b = bb[k] < 0 ? 0 : bb[k];
        const int p = rowpos(T, r);
        if (MODE == MLP_DENSE) {
          v[i0 + k] = ldg16(a.x + uoff(b, p, c8));
        } else if (F8) {
          // the router's MXFP8 copy of the row: 8 E4M3 codes, and the
          // exponent of their 32-column block (every lane of the block loads it)
          const uint32_t row8 = (uint32_t)p * (uint32_t)a.B + (uint32_t)b;
          const uint2 cq = *reinterpret_cast<const uint2*>(a.xq8 + row8 * (uint32_t)W + (uint32_t)c8 * 8u);
          v[i0 + k] = make_uint4(cq.x, cq.y, (uint32_t)a.xe8[row8 * (uint32_t)(W / 32) + (uint32_t)(c8 >> 2)], 0u);
        } else {
          // 32-bit byte offset from the x_hat base (the host keeps that
          // buffer under 4 GiB): one address register per load, which keeps
          // the W = 768 epilogue free of spills
          const uint32_t off = (((uint32_t)p * (uint32_t)a.B + (uint32_t)b) * (uint32_t)W + (uint32_t)c8 * 8u) * 2u;
          v[i0 + k] = ldg16_nt(reinterpret_cast<const char*>(a.xhat) + off);
        }
      }
      if constexpr (IOB == NPRO) {
#pragma unroll
        for (int k = 0; k < IOB; ++k)
          if (bb[k] < 0) v[i0 + k] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // x rows -> LDS x_hat; for DENSE the RMS statistics reduce across the lanes
  // of a row before x_hat is written (RMSNorm in fp32, rho to bf16:
  // TokenMixer-Large section 2.3.3)
  auto store_x = [&](int tix, uint4* v, const float* lgain) {
    if constexpr (F8) {
      // DENSE: RMSNorm in fp32 (the row's U8 units sit in U8 consecutive
      // lanes), then MXFP8 per 32-column block: the block's 4 units sit in 4
      // consecutive lanes (units are numbered row by row, and NT and U8 are
      // multiples of 4). ROUTED / SHARED rows arrive normalised and
      // quantised the same way by the router.
      static_assert(!F8 || (MODE == MLP_DENSE ? (LANE_COL && (U8 == 32 || U8 == 64)) : (U8 % 4 == 0 && NT % 4 == 0)),
                    "F8 row layout");
#pragma unroll
      for (int i = 0; i < NPRO; ++i) {
        int r, c8;
        unit_rc(tix, i, r, c8);
        const int blk = c8 >> 2, st = blk >> 1;
        uint8_t* const scl = &xsc8[r * XSCB + ((st >> 2) * 2 + (blk & 1)) * 4 + (st & 3)];
        if constexpr (MODE != MLP_DENSE) {
          // quantised by the router: codes in .x, .y, the block exponent in .z
          *reinterpret_cast<uint2*>(&xs8[r * XSB + c8 * 8]) = make_uint2(v[i].x, v[i].y);
          if ((c8 & 3) == 0) *scl = (uint8_t)v[i].z;
          continue;
        }
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[i]);
        float n[8], am = 0.f;
        if constexpr (MODE == MLP_DENSE) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = bf2f(h[e]);
            acc += f * f;
          }
#pragma unroll
          for (int o = U8 / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
          const float rinv = 1.0f / sqrtf(acc / (float)W + a.eps);
#pragma unroll
          for (int e = 0; e < 8; ++e) n[e] = bf2f(h[e]) * rinv * lgain[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) n[e] = bf2f(h[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(n[e]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        am = fmaxf(am, __shfl_xor(am, 2, 64));
        const int k = mx_exp(am);
        const float sc = ldexpf(1.f, -k);
        uint2 q;
        q.x = e4m3x4(n[0], n[1], n[2], n[3], sc);
        q.y = e4m3x4(n[4], n[5], n[6], n[7], sc);
        *reinterpret_cast<uint2*>(&xs8[r * XSB + c8 * 8]) = q;
        if ((c8 & 3) == 0) *scl = (uint8_t)(k + 127);
      }
      __syncthreads();
      return;
    }
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
        int r, c8;
        unit_rc(tix, i, r, c8);
        const float rinv = 1.0f / sqrtf(ss[i] / (float)W + a.eps);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[i]);
        float n[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) n[e] = bf2f(h[e]) * rinv * (LANE_COL ? lgain[e] : a.gain[c8 * 8 + e]);
        v[i].x = pack_bf16x2(n[0], n[1]);
        v[i].y = pack_bf16x2(n[2], n[3]);
        v[i].z = pack_bf16x2(n[4], n[5]);
        v[i].w = pack_bf16x2(n[6], n[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < NPRO; ++i) {
      int r, c8;
      unit_rc(tix, i, r, c8);
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
  // F8 at W = 256: the tile's weight scale records (a.wrec dwords per lane
  // and wave) go from global memory straight into LDS (no registers), 16
  // bytes per lane and load: dword d of lane l lands at wsc8 + ((wave RECX /
  // 4 + d / 4) 64 + l) 4 + d % 4, a region only this wave reads. They share
  // bytes with the epilogue's staged tile, so they are issued once the
  // staging has been read; the main loop waits for them.
  auto dma_wrec = [&](const Tile& T) __attribute__((always_inline)) {
    if constexpr (F8 && !REC_REG) {
      const uint4* p = reinterpret_cast<const uint4*>(a.wsc + (((size_t)T.group * 4 + wave) * 64 + lane) * a.wrec);
      for (int m = 0; m < a.wrec / 4; ++m)
        __builtin_amdgcn_global_load_lds(p + m, wsc8 + (wave * (RECX / 4) + m) * 64 * 4, 16, 0, 0);
    }
  };

  // F8 from W = 512: this lane's scale record of a tile's expert / position,
  // and the DWX scale dwords of matrix m (0 gate, 1 up, 2 down) of hidden
  // chunk cc in the tile's chunk order (rotation rot)
  struct Sc {
    uint32_t w[F8 ? DWX : 1];
  };
  auto rec_of = [&](const Tile& T) __attribute__((always_inline)) -> const uint32_t* {
    return a.wsc + (((size_t)T.group * 4 + wave) * 64 + lane) * a.wrec;
  };
  auto gscale = [&](const uint32_t* rec, int rot, int cc, int m) __attribute__((always_inline)) -> Sc {
    cc += rot;
    if (cc >= NC) cc -= NC;
    Sc r;
#pragma unroll
    for (int q = 0; q < (F8 ? DWX : 1); ++q) r.w[q] = rec[(cc * 3 + m) * DWX + q];
    return r;
  };

  // residual rows of the tile, same unit order as load_x
  auto load_resid = [&](int tix, int buf, const Tile& T, uint4* rv) {
#pragma unroll
    for (int i0 = 0; i0 < NPRO; i0 += IOB) {
      int bb[IOB];
#pragma unroll
      for (int k = 0; k < IOB; ++k) {
        int r, c8;
        unit_rc(tix, i0 + k, r, c8);
        bb[k] = rowb[buf][r];
      }
#pragma unroll
      for (int k = 0; k < IOB; ++k) {
        int r, c8;
        unit_rc(tix, i0 + k, r, c8);
        rv[i0 + k] = ldg16(a.resid + uoff(bb[k] < 0 ? 0 : bb[k], rowpos(T, r), c8));
      }
      if constexpr (IOB == NPRO) {
#pragma unroll
        for (int k = 0; k < IOB; ++k)
          if (bb[k] < 0) rv[i0 + k] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // ---- phase shift ----------------------------------------------------------------
  // (set for the shared-expert launch: its alike tiles would otherwise keep
  // every workgroup's HBM-bound epilogue in step; see the host launch)
  // (with two workgroups per CU: the second dispatch round, which the
  // dispatcher places beside the first round's workgroups)
  const bool late = OCC == 2 ? blockIdx.x >= gridDim.x / 2 : ((blockIdx.x >> 3) & 1);
  if (a.stagger > 0 && late) {
    const long long t0 = clock64();
    while (clock64() - t0 < a.stagger) __builtin_amdgcn_s_sleep(16);
  }

  // ---- first tile ---------------------------------------------------------------
  Tile cur, nx;
  uint4 kx[RESX ? NPRO : 1];   // RESX: raw input rows of the current tile
  int ci = 0, ni = 0;
  bool has_nx;
  if constexpr (MODE == MLP_ROUTED) {
    __shared__ int qfirst[2];
    if (tid == 0) {
      // the second claim goes out only once the first has returned: the
      // workgroups starting together then take queue entries w and about
      // w + grid, not w and w + 1, so the tiles in flight at any time are
      // consecutive entries (few experts' weights live at once)
      const int q0 = atomicAdd(&a.qhead[qx], 1);
      asm volatile("" ::"v"(q0));
      qfirst[0] = q0;
      qfirst[1] = atomicAdd(&a.qhead[qx], 1);
    }
    __syncthreads();
    if (!qdecode(qfirst[0], cur)) return;                      // uniform per workgroup
    has_nx = qdecode(qfirst[1], nx);
  } else {
    ci = next_valid(blockIdx.x, cur);
    if (ci >= total) return;                                   // uniform per workgroup
    ni = next_valid(ci + gridDim.x, nx);
    has_nx = ni < total;
  }
  int buf = 0;
  set_rows(cur, 0);
  cw = bind(cur);
  nw = has_nx ? bind(nx) : cw;
  // REC_REG: the gate / up scales of the tile's first chunk, loaded with
  // (or, for later tiles, ahead of) its first weight fragments
  Sc g0{}, u0{};
  __syncthreads();                         // row table visible
  {
    // the first rows go out before the weight ring: a wave's loads retire
    // in order, so the normalisation below waits for the rows only
    uint4 v[NPRO];
    float g[8];
    load_gain(g);
    load_x(tid, 0, cur, v);
    dma_wrec(cur);
    if constexpr (REC_REG) {
      g0 = gscale(rec_of(cur), cw.rot, 0, 0);
      u0 = gscale(rec_of(cur), cw.rot, 0, 1);
    }
    if constexpr (F8) {
#pragma unroll
      for (int f = 0; f < NFR8; ++f) issue_frag8(ring8[f], cw, 0, f);
    } else if constexpr (NW == 4) {
#pragma unroll
      for (int f = 0; f < NFR; ++f) issue_frag(fslot(f), cw, 0, f);
    } else {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) issue(ring[s], cw, 0, s);
    }
    if constexpr (RESX) {
#pragma unroll
      for (int i = 0; i < NPRO; ++i) kx[i] = v[i];
    }
    store_x(tid, v, g);
  }

  while (true) {
    // ROUTED: the next tile's bucket entry of row tid, loaded now so that its
    // latency is spent under this tile's main loop
    int nent = 0;
    if constexpr (MODE == MLP_ROUTED)
      if (has_nx && tid < nx.nrows) nent = a.rows[(size_t)nx.p * a.B * a.top_k + nx.start + tid];
    // ROUTED: the next tile's row table from that entry, its gates, and the
    // claim of the tile after next. The compiler cannot follow the entry's
    // load across the main loop and waits for every load in flight at its
    // first use, so 4-wave tiles run this before the postamble, while only
    // the tile's own (warm) fragments are in flight -- not after it, when
    // the next tile's first fragments (often a cold expert) are. Every
    // thread issues the gate load (padding rows and threads past BM read
    // entry 0 and never use it): a load on one path only makes the compiler
    // drain every load in flight where the paths join. The gate and the
    // claimed slot go to LDS after the epilogue (only the next epilogue
    // reads them).
    float ngate = 0.f;
    int qs = 0;
    auto routed_setup = [&]() __attribute__((always_inline)) {
      const bool ok = has_nx && tid < BM && tid < nx.nrows;
      const int b = ok ? nent / a.top_k : -1;
      const int gi = ok ? (b * a.P + nx.p) * a.top_k + (nent - b * a.top_k) : 0;
      ngate = a.gate[gi];
      if (has_nx && tid < BM) {
        rowb[buf ^ 1][tid] = b;
        rowgi[buf ^ 1][tid] = gi;
      }
      if (has_nx && tid == 0) qs = atomicAdd(&a.qhead[qx], 1);
    };

    // ---- main loop ---------------------------------------------------------------
    f32x16 oacc[RBW][NBO];
    // (TP clears them where its GEMM2 phase starts: cleared here they
    // would stay live through the GEMM1 phase)
    if constexpr (!TP) {
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < NBO; ++j) oacc[i][j] = f32x16{};
    }

    if constexpr (NW == 8) {
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
          if (s == YS) {
            __syncthreads();                                         // barrier Y
            // this group computes U before its next barrier: its MFMAs issue
            // ahead of the other group's, so that its SiLU runs while the
            // other group's MFMAs keep the pipe busy (the arbiter otherwise
            // favours the older waves, group A, in both halves)
            __builtin_amdgcn_s_setprio(2);
          }
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
        __builtin_amdgcn_s_setprio(0);

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
    } else if constexpr (F8) {
      // MXFP8 on 32x32x64 scaled MFMAs. Dense sub-layers: the chunk schedule
      // of the 4-wave kernel below (GEMM1(i); GEMM2(i-1) with U(i) between
      // its MFMAs; barrier). MoE modes (TP): the two-phase tile (tp_tile).
      // GEMM1 step s reads 64 columns of x_hat codes and the rows' scale
      // words (byte s % 4 of word s / 4), GEMM2 step t 64 hidden units of U
      // codes and their scales; the weight scales come from the tile's
      // records in LDS (W = 256) or straight from global memory (REC_REG).
      f32x16 sg[RBW], su[RBW];
      uint32_t xsw[RBW][DWX];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int q = 0; q < DWX; ++q)
          xsw[rb][q] = *reinterpret_cast<const uint32_t*>(&xsc8[(rb * 32 + l32) * XSCB + (2 * q + h32) * 4]);
      const int rot = cw.rot;
      // W = 256: the scale records' LDS writes (global_load_lds, counted
      // like loads)
      if constexpr (!REC_REG) __builtin_amdgcn_s_waitcnt(0);
      const uint32_t* const rec = rec_of(cur);
      // scale dwords of matrix m (0 gate, 1 up, 2 down) of chunk cc: from
      // the LDS records (W = 256)
      auto wscale = [&](int cc, int m) __attribute__((always_inline)) -> Sc {
        cc += rot;
        if (cc >= NC) cc -= NC;
        Sc r;
#pragma unroll
        for (int q = 0; q < DWX; ++q) {
          const int dw = (cc * 3 + m) * DWX + q;
          r.w[q] = wsc8[((wave * (RECX / 4) + (dw >> 2)) * 64 + lane) * 4 + (dw & 3)];
        }
        return r;
      };
      auto read_xb = [&](i32x8* dst, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const uint8_t* q = xs8 + (rb * 32 + l32) * XSB + st * 64 + 16 * h32;
          dst[rb] = join8(*reinterpret_cast<const uint4*>(q), *reinterpret_cast<const uint4*>(q + 32));
        }
      };
      auto read_ub = [&](i32x8* dst, int ubuf, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const uint8_t* q = us8 + ubuf * BM * USB + (rb * 32 + l32) * USB + t * 64 + 16 * h32;
          dst[rb] = join8(*reinterpret_cast<const uint4*>(q), *reinterpret_cast<const uint4*>(q + 32));
        }
      };
      // U of row block rb: rho_fp8(silu(gate) * up) with one scale per row
      // and this wave's 32 hidden units (16 in this lane, 16 in lane ^ 32)
      // in two halves (8 values each, the second also quantises and stores),
      // so that a GEMM2 step can place MFMAs between them; `am` carries the
      // running block maximum from the first half to the second
      auto u_half8 = [&](int ubuf, int rb, int part, float& am) __attribute__((always_inline)) {
        f32x16& u = sg[rb];   // the gate accumulator is dead once U is formed
        if (part == 0) am = 0.f;
#pragma unroll
        for (int v = 8 * part; v < 8 * part + 8; ++v) {
          u[v] = silu_fast(u[v]) * su[rb][v];
          am = fmaxf(am, fabsf(u[v]));
        }
        if (part == 0) return;
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        const int k = mx_exp(am);
        const float sc = ldexpf(1.f, -k);
        uint8_t* row = us8 + ubuf * BM * USB + (rb * 32 + l32) * USB + wc * 32 + 4 * h32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint32_t*>(row + 8 * g4) = e4m3x4(u[4 * g4], u[4 * g4 + 1], u[4 * g4 + 2], u[4 * g4 + 3], sc);
        if (h32 == 0) usc8[ubuf * BM * 8 + (rb * 32 + l32) * 8 + (wc & 1) * 4 + (wc >> 1)] = (uint8_t)(k + 127);
      };
      auto u_group8 = [&](int ubuf, int rb) __attribute__((always_inline)) {
        float am;
        u_half8(ubuf, rb, 0, am);
        __builtin_amdgcn_sched_barrier(0);
        u_half8(ubuf, rb, 1, am);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto gemm1_8 = [&](auto refill_at, const Sc& gsc, const Sc& usc) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          sg[i] = f32x16{};
          su[i] = f32x16{};
        }
        i32x8 xb[2][RBW];
#pragma unroll
        for (int st = 0; st < KS8; ++st) {
          read_xb(xb[st & 1], st);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            sg[rb] = mfma8s(st & 3, st & 3, ring8[(2 * st) % NFR8], xb[st & 1][rb], gsc.w[st >> 2],
                            xsw[rb][st >> 2], sg[rb]);
            su[rb] = mfma8s(st & 3, st & 3, ring8[(2 * st + 1) % NFR8], xb[st & 1][rb], usc.w[st >> 2],
                            xsw[rb][st >> 2], su[rb]);
          }
          refill_at(ring8[(2 * st) % NFR8], 2 * st + NFR8);
          refill_at(ring8[(2 * st + 1) % NFR8], 2 * st + 1 + NFR8);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // GEMM2 of a chunk from U buffer rbuf; with_u: U(next chunk) row block
      // t goes to buffer wbuf after step t's MFMAs
      auto gemm2_8 = [&](int rbuf, int wbuf, auto with_u_tag, auto refill_at, auto pos0_tag, const Sc& dsc)
          __attribute__((always_inline)) {
        constexpr bool with_u = decltype(with_u_tag)::value;
        constexpr int pos0 = decltype(pos0_tag)::value;
        static_assert(RBW == TS8, "one U row block per GEMM2 step");
        uint32_t usw[RBW];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
          usw[rb] = *reinterpret_cast<const uint32_t*>(&usc8[rbuf * BM * 8 + (rb * 32 + l32) * 8 + h32 * 4]);
        i32x8 ub[2][RBW];
#pragma unroll
        for (int t = 0; t < TS8; ++t) {
          read_ub(ub[t & 1], rbuf, t);
          __builtin_amdgcn_sched_barrier(0);
          // row block 0's MFMAs, U half 0, row block 1's MFMAs, U half 1
          float am;
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
            for (int j = 0; j < NBO; ++j)
              oacc[rb][j] = mfma8s((j * 2 + t) & 3, t, ring8[(pos0 + t * NBO + j) % NFR8], ub[t & 1][rb],
                                   dsc.w[(j * 2 + t) >> 2], usw[rb], oacc[rb][j]);
            if constexpr (with_u) {
              u_half8(wbuf, t, rb, am);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int j = 0; j < NBO; ++j) refill_at(ring8[(pos0 + t * NBO + j) % NFR8], pos0 + t * NBO + j + NFR8);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // REC_REG: the scales of the next GEMM phases, loaded one phase ahead:
      // gate / up of chunk i + 1 and down of chunk i go out as chunk i
      // starts (ng, nu, nd), ahead of that chunk's weight refills
      Sc ng{}, nu{}, nd{};
      auto chunk_loop8 = [&](auto more_tag) __attribute__((always_inline)) {
        constexpr bool MORE = decltype(more_tag)::value;
        Sc cg, cu;
        if constexpr (REC_REG) {
          cg = g0;
          cu = u0;
          if constexpr (MORE) {
            ng = gscale(rec, rot, 1, 0);
            nu = gscale(rec, rot, 1, 1);
          }
          nd = gscale(rec, rot, 0, 2);
        } else {
          cg = wscale(0, 0);
          cu = wscale(0, 1);
        }
        gemm1_8([&](i32x8& dst, int k2) __attribute__((always_inline)) {
                  if (k2 < F1)
                    issue_frag8(dst, cw, 0, k2);
                  else if (MORE)
                    issue_frag8(dst, cw, 1, k2 - F1);
                  else
                    issue_frag8(dst, cw, 0, k2);
                },
                cg, cu);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) u_group8(0, rb);
        __syncthreads();
        auto iteration = [&](int i, auto last_tag) __attribute__((always_inline)) {
          constexpr bool LAST = decltype(last_tag)::value;
          auto refill_at = [&](i32x8& dst, int k2) __attribute__((always_inline)) {
            if (k2 < F1) {
              issue_frag8(dst, cw, i, k2);
            } else if (k2 < FS) {
              issue_frag8(dst, cw, i - 1, k2);
            } else if (!LAST) {
              issue_frag8(dst, cw, i + 1, k2 - FS);
            } else {
              issue_frag8(dst, cw, NC - 1, k2 - FS + F1);
            }
          };
          Sc ig, iu, id;
          if constexpr (REC_REG) {
            ig = ng;
            iu = nu;
            id = nd;
            if constexpr (!LAST) {
              ng = gscale(rec, rot, i + 1, 0);
              nu = gscale(rec, rot, i + 1, 1);
            }
            nd = gscale(rec, rot, i, 2);
          } else {
            ig = wscale(i, 0);
            iu = wscale(i, 1);
            id = wscale(i - 1, 2);
          }
          gemm1_8(refill_at, ig, iu);
          gemm2_8((i - 1) & 1, i & 1, std::true_type{}, refill_at, std::integral_constant<int, F1>{}, id);
          __syncthreads();
        };
        if constexpr (MORE) {
          for (int i = 1; i + 1 < NC; ++i) iteration(i, std::integral_constant<bool, false>{});
          iteration(NC - 1, std::integral_constant<bool, true>{});
        }
        if constexpr (MODE == MLP_ROUTED) routed_setup();
        Sc dsc;
        if constexpr (REC_REG) {
          dsc = nd;
          // the next tile's first gate / up scales, ahead of its first
          // weight fragments (after the last tile: this tile's, unused --
          // loads on one path only would drain every load in flight where
          // the paths join)
          const uint32_t* const nrec = rec_of(has_nx ? nx : cur);
          g0 = gscale(nrec, nw.rot, 0, 0);
          u0 = gscale(nrec, nw.rot, 0, 1);
        } else {
          dsc = wscale(NC - 1, 2);
        }
        gemm2_8((NC - 1) & 1, 0, std::false_type{},
                [&](i32x8& dst, int k2) __attribute__((always_inline)) {
                  if (k2 < F2) issue_frag8(dst, cw, NC - 1, F1 + k2);
                  else issue_frag8(dst, nw, 0, k2 - F2);
                },
                std::integral_constant<int, 0>{}, dsc);
      };
      // TP: U of chunk c, row block rb, into the whole-hidden U tile: one
      // scale per row and 32 hidden units (this wave's block 4c + wc; 16
      // values in this lane, 16 in lane ^ 32)
      auto u_tp = [&](int c, int rb) __attribute__((always_inline)) {
        f32x16& u = sg[rb];
        float am = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          u[v] = silu_fast(u[v]) * su[rb][v];
          am = fmaxf(am, fabsf(u[v]));
        }
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        const int k = mx_exp(am);
        const float sc = ldexpf(1.f, -k);
        uint8_t* row = us8 + (rb * 32 + l32) * USBA + c * HC + wc * 32 + 4 * h32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint32_t*>(row + 8 * g4) = e4m3x4(u[4 * g4], u[4 * g4 + 1], u[4 * g4 + 2], u[4 * g4 + 3], sc);
        const int blk = c * 4 + wc, T = blk >> 1;
        if (h32 == 0) usc8[(rb * 32 + l32) * USCB + ((T >> 2) * 2 + (blk & 1)) * 4 + (T & 3)] = (uint8_t)(k + 127);
      };
      // TP: GEMM2 of chunk c over the whole-hidden U tile; step T = 2c + t
      // of the hidden reads its U scales from the row's scale words (byte T
      // % 4 shifted down: T is not a compile-time constant)
      auto gemm2_tp = [&](int c, auto refill_at, const Sc& dsc) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < TS8; ++t) {
          const int T = c * TS8 + t;
          uint32_t usw[RBW];
          i32x8 ub[RBW];
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            const int row = rb * 32 + l32;
            usw[rb] = *reinterpret_cast<const uint32_t*>(&usc8[row * USCB + ((T >> 2) * 2 + h32) * 4]) >> (8 * (T & 3));
            const uint8_t* q = us8 + row * USBA + T * 64 + 16 * h32;
            ub[rb] = join8(*reinterpret_cast<const uint4*>(q), *reinterpret_cast<const uint4*>(q + 32));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int j = 0; j < NBO; ++j)
              oacc[rb][j] = mfma8s((j * 2 + t) & 3, 0, ring8[(t * NBO + j) % NFR8], ub[rb], dsc.w[(j * 2 + t) >> 2],
                                   usw[rb], oacc[rb][j]);
#pragma unroll
          for (int j = 0; j < NBO; ++j) refill_at(ring8[(t * NBO + j) % NFR8], t * NBO + j + NFR8);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // TP tile: the weight stream runs GEMM1 fragments of chunks 0 .. NC-1,
      // then GEMM2 fragments of chunks 0 .. NC-1, then the next tile's.
      // Scales one chunk ahead, as in the chunk pipeline.
      auto tp_tile = [&]() __attribute__((always_inline)) {
        Sc ng = g0, nu = u0, nd{};
        auto p1 = [&](int c, auto last_tag) __attribute__((always_inline)) {
          constexpr bool LASTC = decltype(last_tag)::value;
          const Sc g = ng, u = nu;
          if constexpr (!LASTC) {
            ng = gscale(rec, rot, c + 1, 0);
            nu = gscale(rec, rot, c + 1, 1);
          } else {
            nd = gscale(rec, rot, 0, 2);
          }
          gemm1_8([&](i32x8& dst, int k2) __attribute__((always_inline)) {
                    if (k2 < F1) issue_frag8(dst, cw, c, k2);
                    else if (!LASTC) issue_frag8(dst, cw, c + 1, k2 - F1);
                    else issue_frag8(dst, cw, 0, k2);          // GEMM2 fragment k2 - F1 of chunk 0
                  },
                  g, u);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) u_tp(c, rb);
        };
        for (int c = 0; c + 1 < NC; ++c) p1(c, std::false_type{});
        p1(NC - 1, std::true_type{});
        __syncthreads();                                     // the whole U tile written
        if constexpr (MODE == MLP_ROUTED) routed_setup();
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
          for (int j = 0; j < NBO; ++j) oacc[i][j] = f32x16{};
        auto p2 = [&](int c, auto last_tag) __attribute__((always_inline)) {
          constexpr bool LASTC = decltype(last_tag)::value;
          const Sc d = nd;
          if constexpr (!LASTC) {
            nd = gscale(rec, rot, c + 1, 2);
          } else {
            // the next tile's first gate / up scales (after the last tile:
            // this tile's, unused)
            const uint32_t* const nrec = rec_of(has_nx ? nx : cur);
            g0 = gscale(nrec, nw.rot, 0, 0);
            u0 = gscale(nrec, nw.rot, 0, 1);
          }
          gemm2_tp(c,
                   [&](i32x8& dst, int k2) __attribute__((always_inline)) {
                     if (k2 < F2) issue_frag8(dst, cw, c, F1 + k2);
                     else if (!LASTC) issue_frag8(dst, cw, c + 1, F1 + k2 - F2);
                     else issue_frag8(dst, nw, 0, k2 - F2);
                   },
                   d);
        };
        for (int c = 0; c + 1 < NC; ++c) p2(c, std::false_type{});
        p2(NC - 1, std::true_type{});
      };
      if constexpr (TP)
        tp_tile();
      else if (NC > 1)
        chunk_loop8(std::true_type{});
      else
        chunk_loop8(std::false_type{});
    } else {
      // One wave per SIMD: every wave runs all BM rows, and the VALU work
      // (silu(gate) * up) is software-pipelined against the MFMAs instead of
      // against a second wave. Chunk schedule, i = hidden chunk:
      //   preamble   GEMM1(0); U(0) -> U buffer 0; barrier
      //   iteration  GEMM1(i); GEMM2(i-1) with U(i) -> buffer i&1 computed
      //              between its MFMAs; barrier                 (0 < i < NC)
      //   postamble  GEMM2(NC-1)
      // GEMM2(i-1) reads buffer (i-1)&1, complete since the previous
      // barrier; buffer i&1 was last read by GEMM2(i-2), before it. The
      // weight stream follows the same order, into the next tile's preamble.
      f32x16 sg[RBW], su[RBW];
      uint4 xa[2][RBW];
      uint4 ua[2][RBW];
      constexpr int SPS = RBW * 4 / S2;        // U groups (4 hidden units) per GEMM2 step
      static_assert((RBW * 4) % S2 == 0, "U groups must spread evenly over GEMM2 steps");
      auto read_xa = [&](uint4* dst, int q) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
          dst[rb] = *reinterpret_cast<const uint4*>(&xs[(rb * 32 + l32) * XS + q * 16 + h32 * 8]);
      };
      auto read_ua = [&](uint4* dst, const uint16_t* ub, int t) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
          dst[rb] = *reinterpret_cast<const uint4*>(&ub[(rb * 32 + l32) * US + t * 16 + h32 * 8]);
      };
      // U group gi (row block gi/4, hidden units 8*(gi%4) + 4*h32 + 0..3 of
      // this wave's 32): rho(silu(gate) * up), one 8-byte LDS store
      auto u_group = [&](uint16_t* ub, int gi) __attribute__((always_inline)) {
        const int rb = gi >> 2, g4 = gi & 3;
        float uv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[e] = silu_fast(sg[rb][4 * g4 + e]) * su[rb][4 * g4 + e];
        uint2 w2;
        w2.x = pack_bf16x2(uv[0], uv[1]);
        w2.y = pack_bf16x2(uv[2], uv[3]);
        *reinterpret_cast<uint2*>(&ub[(rb * 32 + l32) * US + wc * 32 + 8 * g4 + 4 * h32]) = w2;
      };
      // GEMM1 of chunk c over S1 k-steps; `refill_at(slot, k)` loads the
      // fragment at position k of the segment's stream (k >= NFR: past the
      // consumed one by a full ring) and `last` (the final step) may
      // prefetch the first GEMM2 operands
      auto gemm1 = [&](auto refill_at, auto at_last) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          sg[i] = f32x16{};
          su[i] = f32x16{};
        }
        read_xa(xa[0], 0);
#pragma unroll
        for (int q = 0; q < S1; ++q) {
          if (q + 1 < S1) read_xa(xa[(q + 1) & 1], q + 1);
          else at_last();
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            sg[rb] = mfma32(fslot(2 * q), xa[q & 1][rb], sg[rb]);
            su[rb] = mfma32(fslot(2 * q + 1), xa[q & 1][rb], su[rb]);
          }
          refill_at(fslot(2 * q), 2 * q + NFR);
          refill_at(fslot(2 * q + 1), 2 * q + 1 + NFR);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // GEMM2 of one chunk from U buffer `ub` (its first operands already in
      // ua[0]); with `with_u` the next chunk's U groups go to `ubw` between
      // the MFMAs, SPS groups per k-step
      auto gemm2 = [&](const uint16_t* ub, uint16_t* ubw, auto with_u_tag, auto refill_at, auto pos0_tag)
          __attribute__((always_inline)) {
        constexpr bool with_u = decltype(with_u_tag)::value;
        constexpr int pos0 = decltype(pos0_tag)::value;   // first fragment's segment position
#pragma unroll
        for (int t = 0; t < S2; ++t) {
          if (t + 1 < S2) read_ua(ua[(t + 1) & 1], ub, t + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int j = 0; j < NBO; ++j)
              oacc[rb][j] = mfma32(fslot(pos0 + NBO * t + j), ua[t & 1][rb], oacc[rb][j]);   // O^T block
          if constexpr (with_u) {
#pragma unroll
            for (int k = 0; k < SPS; ++k) u_group(ubw, t * SPS + k);
          }
#pragma unroll
          for (int j = 0; j < NBO; ++j) refill_at(fslot(pos0 + NBO * t + j), pos0 + NBO * t + j + NFR);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // The whole chunk loop comes in two copies, for one chunk and for more:
      // the preamble's look-ahead reads GEMM1(1) fragments (2 loads per
      // step) or, with a single chunk, GEMM2(0) fragments (NBO loads), and
      // paths that rejoin with different loads in flight make the compiler
      // drain them all (vmcnt(0)) at the join.
      auto chunk_loop = [&](auto more_tag) __attribute__((always_inline)) {
        constexpr bool MORE = decltype(more_tag)::value;
        // preamble: segment positions k < F1 are GEMM1(0); beyond, GEMM1(1)
        // of iteration 1, or with a single chunk the postamble's GEMM2(0)
        gemm1([&](uint4& dst, int k2) __attribute__((always_inline)) {
                if (k2 < F1)
                  issue_frag(dst, cw, 0, k2);
                else if (MORE)
                  issue_frag(dst, cw, 1, k2 - F1);
                else
                  issue_frag(dst, cw, 0, k2);
              },
              [] {});
#pragma unroll
        for (int gi = 0; gi < RBW * 4; ++gi) u_group(us, gi);
        __syncthreads();

        // iterations: positions [0, F1) GEMM1(i), [F1, FS) GEMM2(i-1); past
        // FS the next iteration's GEMM1(i+1), or for the last iteration the
        // postamble's GEMM2(NC-1)
        auto iteration = [&](int i, auto last_tag) __attribute__((always_inline)) {
          constexpr bool LAST = decltype(last_tag)::value;
          uint16_t* ubw = us + (i & 1) * BM * US;
          const uint16_t* ubr = us + ((i - 1) & 1) * BM * US;
          auto refill_at = [&](uint4& dst, int k2) __attribute__((always_inline)) {
            if (k2 < F1) {
              issue_frag(dst, cw, i, k2);
            } else if (k2 < FS) {
              issue_frag(dst, cw, i - 1, k2);
            } else if (!LAST) {
              issue_frag(dst, cw, i + 1, k2 - FS);
            } else {
              issue_frag(dst, cw, NC - 1, k2 - FS + F1);
            }
          };
          gemm1(refill_at, [&] { read_ua(ua[0], ubr, 0); });
          gemm2(ubr, ubw, std::true_type{}, refill_at, std::integral_constant<int, F1>{});
          __syncthreads();
        };
        if constexpr (MORE) {
          for (int i = 1; i + 1 < NC; ++i) iteration(i, std::integral_constant<bool, false>{});
          iteration(NC - 1, std::integral_constant<bool, true>{});
        }

        if constexpr (MODE == MLP_ROUTED) routed_setup();
        // postamble: GEMM2(NC-1); past its end the stream enters the next
        // tile's preamble
        {
          const uint16_t* ubr = us + ((NC - 1) & 1) * BM * US;
          read_ua(ua[0], ubr, 0);
          gemm2(ubr, nullptr, std::false_type{},
                [&](uint4& dst, int k2) __attribute__((always_inline)) {
                  if (k2 < F2) issue_frag(dst, cw, NC - 1, F1 + k2);
                  else issue_frag(dst, nw, 0, k2 - F2);
                },
                std::integral_constant<int, 0>{});
        }
      };
      if (NC > 1)
        chunk_loop(std::true_type{});
      else
        chunk_loop(std::false_type{});
    }

    // ---- between tiles: stage O, start the next tile's loads, epilogue --------
    // The ring already holds the next tile's first fragments (see refill).
    const bool has_next = has_nx;
    if constexpr (MODE == MLP_ROUTED) {
      if constexpr (NW == 8) routed_setup();
    } else if (has_next) {
      set_rows(nx, buf ^ 1);
    }
    // an opaque copy of the thread index: keeps the compiler from hoisting
    // the epilogue's and the next prologue's address arithmetic out of the
    // tile loop, where it would stay live through the main loop
    int etid = tid;
    asm volatile("" : "+v"(etid));
    // EARLY: with at most 16 row units per lane the epilogue's row loads go
    // out before the staging (their registers are free then); at W = 768
    // (24 units, all accumulators in use until staged) they wait for the
    // last part, and the residual is loaded beside each batch of units
    constexpr bool EARLY = NPRO <= 16;
    constexpr bool PREF_R = (MODE != MLP_ROUTED) && (EARLY || NPART == 1);
    constexpr int PR = BM / NPART;           // rows per staged part
    constexpr int NE = PR * U8 / NT;         // units per lane per part
    static_assert((PR * U8) % NT == 0, "part units must divide evenly");
    uint4 pr[PREF_R && !RESX ? NPRO : 1];
    // Defined on every path: a conditionally written px becomes a value
    // carried around the tile loop and stays live through the main loop.
    // 4-wave ROUTED tiles with up to 16 units per lane leave it undefined
    // off the has_next path (it is read only on that path): there the
    // clearing writes made the compiler wait for every load in flight, the
    // next tile's first weight fragments included, before the epilogue.
    // (At W = 768 an undefined px is kept in scratch memory instead.)
    uint4 px[NPRO];
    float pg[8];
    if constexpr (MODE != MLP_ROUTED || NW == 8 || !EARLY) {
#pragma unroll
      for (int i = 0; i < NPRO; ++i) px[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) pg[e] = 0.f;
    }
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      __syncthreads();
      if (part == (EARLY ? 0 : NPART - 1)) {
        // the residual rows and the next tile's x rows do not depend on the
        // staged accumulators: they go out first, after the barrier above
        // (which also makes the next tile's row table visible)
        if constexpr (PREF_R && !RESX) load_resid(etid, buf, cur, pr);
        if (has_next) {
          load_gain(pg);
          load_x(etid, buf ^ 1, nx, px);
        }
      }
      if (NPART == 1 || NW == 4 || wr == part) {
        // C layout of an O^T block (32 columns x 32 rows): lane holds row l32
        // and columns 8*(v/4) + 4*h32 + v%4 -> 4 consecutive columns per v-group
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          // parts of 4-wave tiles are row blocks: part p stages block p
          if (NW == 4 && NPART > 1 && rb != part) continue;
#pragma unroll
          for (int j = 0; j < NBO; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int r = (NPART == 1 ? row0 + rb * 32 : (NW == 4 ? 0 : rb * 32)) + l32;
              const int col = (wc * NBO + j) * 32 + 8 * g4 + 4 * h32;
              *reinterpret_cast<float4*>(&stage[r * SS + col]) =
                  make_float4(oacc[rb][j][4 * g4], oacc[rb][j][4 * g4 + 1], oacc[rb][j][4 * g4 + 2],
                              oacc[rb][j][4 * g4 + 3]);
            }
        }
      }
      __syncthreads();
      // O goes out of LDS in 16-byte units: residual / extra / output through
      // the row map, gated expert outputs as bf16 rows. Units go in batches
      // of UB whose global loads (partials, extra) are all issued before any
      // is consumed, so a lane keeps several loads in flight.
      constexpr int UB = (NW == 4 && NE % 4 == 0) ? 4 : (NE % 2 == 0) ? 2 : 1;
#pragma unroll
      for (int i0 = 0; i0 < NE; i0 += UB) {
        float o[UB][8];
        int bu[UB], pu[UB], c8u[UB], Ru[UB];
#pragma unroll
        for (int k = 0; k < UB; ++k) {
          int r;
          unit_rc(etid, i0 + k, r, c8u[k]);
          Ru[k] = part * PR + r;
          bu[k] = rowb[buf][Ru[k]];
          pu[k] = rowpos(cur, Ru[k]);
          const float4 o0 = *reinterpret_cast<const float4*>(&stage[r * SS + c8u[k] * 8]);
          const float4 o1 = *reinterpret_cast<const float4*>(&stage[r * SS + c8u[k] * 8 + 4]);
          o[k][0] = o0.x; o[k][1] = o0.y; o[k][2] = o0.z; o[k][3] = o0.w;
          o[k][4] = o1.x; o[k][5] = o1.y; o[k][6] = o1.z; o[k][7] = o1.w;
        }
        if constexpr (MODE == MLP_ROUTED) {
#pragma unroll
          for (int k = 0; k < UB; ++k) {
            if (bu[k] < 0) continue;
            const float g = rowg[buf][Ru[k]];
            uint4 w;
            w.x = pack_bf16x2(g * o[k][0], g * o[k][1]);
            w.y = pack_bf16x2(g * o[k][2], g * o[k][3]);
            w.z = pack_bf16x2(g * o[k][4], g * o[k][5]);
            w.w = pack_bf16x2(g * o[k][6], g * o[k][7]);
            stg16_nt(a.part + (size_t)rowgi[buf][Ru[k]] * W + c8u[k] * 8, w);
          }
        } else {
          // At W = 768 the expert-output and residual loads are
          // unconditional (rows past the tile end read row 0, slots past
          // top_k read slot 0; those values are not used): a load on one
          // path only makes the compiler wait for every load in flight where
          // the paths join -- the next tile's weight fragments included. (At
          // W <= 512 that measured slower.) The inter-residual is loaded
          // only by the RV_EXTRA instantiation, unconditionally.
          if constexpr (MODE == MLP_SHARED) {
            // the routed experts' gated outputs, four slots at a time
            for (int s0 = 0; s0 < a.top_k; s0 += 4) {
              uint4 q[UB][4];
#pragma unroll
              for (int k = 0; k < UB; ++k)
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                  if constexpr (EARLY) {
                    q[k][sl] = make_uint4(0, 0, 0, 0);
                    if (bu[k] >= 0 && s0 + sl < a.top_k)
                      q[k][sl] = ldg16(a.part + (((size_t)bu[k] * a.P + pu[k]) * a.top_k + s0 + sl) * W + c8u[k] * 8);
                  } else {
                    const int bq = bu[k] < 0 ? 0 : bu[k];
                    const int sq = s0 + sl < a.top_k ? s0 + sl : 0;
                    q[k][sl] = ldg16_nt(a.part + (((size_t)bq * a.P + pu[k]) * a.top_k + sq) * W + c8u[k] * 8);
                  }
                }
#pragma unroll
              for (int k = 0; k < UB; ++k)
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                  if (s0 + sl >= a.top_k) continue;
                  const uint16_t* qh = reinterpret_cast<const uint16_t*>(&q[k][sl]);
#pragma unroll
                  for (int e = 0; e < 8; ++e) o[k][e] += bf2f(qh[e]);
                }
            }
          }
          int64_t off[UB];
          uint4 ev[UB], rv[UB];
#pragma unroll
          for (int k = 0; k < UB; ++k) {
            off[k] = uoff(bu[k] < 0 ? 0 : bu[k], pu[k], c8u[k]);
            ev[k] = make_uint4(0, 0, 0, 0);
            if constexpr (EXTRA) ev[k] = ldg16(a.extra + off[k]);
            if constexpr (!PREF_R) rv[k] = ldg16(a.resid + off[k]);
          }
#pragma unroll
          for (int k = 0; k < UB; ++k) {
            if (bu[k] < 0) continue;
            uint4 rvv;
            if constexpr (RESX) rvv = kx[part * NE + i0 + k];
            else if constexpr (PREF_R) rvv = pr[part * NE + i0 + k];
            else rvv = rv[k];
            const uint16_t* rh = reinterpret_cast<const uint16_t*>(&rvv);
            const uint16_t* eh = reinterpret_cast<const uint16_t*>(&ev[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[k][e] += bf2f(rh[e]) + bf2f(eh[e]);
            uint4 w;
            w.x = pack_bf16x2(o[k][0], o[k][1]);
            w.y = pack_bf16x2(o[k][2], o[k][3]);
            w.z = pack_bf16x2(o[k][4], o[k][5]);
            w.w = pack_bf16x2(o[k][6], o[k][7]);
            if constexpr (MODE == MLP_SHARED) stg16_nt(a.out + off[k], w);
            else *reinterpret_cast<uint4*>(a.out + off[k]) = w;
          }
        }
      }
    }
    if (!has_next) break;
    if (MODE == MLP_ROUTED && tid < BM) rowg[buf ^ 1][tid] = ngate;
    if (MODE == MLP_ROUTED && tid == 0) qslot = qs;
    __syncthreads();                       // staging reads done before x_hat is rewritten
    const int knext = qslot;
    if constexpr (RESX) {
#pragma unroll
      for (int i = 0; i < NPRO; ++i) kx[i] = px[i];
    }
    dma_wrec(nx);
    store_x(etid, px, pg);
    cur = nx;
    buf ^= 1;
    cw = nw;
    if constexpr (MODE == MLP_ROUTED) {
      has_nx = qdecode(knext, nx);
    } else {
      ci = ni;
      ni = next_valid(ci + gridDim.x, nx);
      has_nx = ni < total;
    }
    nw = has_nx ? bind(nx) : cw;
  }
}

template <int W, int MODE>
void launch_wm(const MlpArgs& a, int grid, hipStream_t s) {
  constexpr int NW = mlp_waves(MODE, W), OCC = mlp_occupancy(MODE, W);
  // Mix: the residual is the input through the same map (the raw rows fit
  // in registers up to W = 512)
  constexpr bool MIX_OK = MODE == MLP_DENSE && W <= 512;
  if (MIX_OK && a.map.mix && !a.extra)
    hipLaunchKernelGGL((mlp_kernel<W, MODE, NW, OCC, MIX_OK ? RV_MIX : RV_PLAIN, false>), dim3(grid), dim3(64 * NW),
                       0, s, a);
  else if (MODE != MLP_ROUTED && a.extra)
    hipLaunchKernelGGL((mlp_kernel<W, MODE, NW, OCC, MODE != MLP_ROUTED ? RV_EXTRA : RV_PLAIN, false>), dim3(grid),
                       dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_kernel<W, MODE, NW, OCC, RV_PLAIN, false>), dim3(grid), dim3(64 * NW), 0, s, a);
}

template <int W>
hipError_t launch_w(int mode, const MlpArgs& a, int grid, hipStream_t s) {
  switch (mode) {
    case MLP_DENSE: launch_wm<W, MLP_DENSE>(a, grid, s); break;
    case MLP_ROUTED: launch_wm<W, MLP_ROUTED>(a, grid, s); break;
    default: launch_wm<W, MLP_SHARED>(a, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace

bool mlp_width_supported(int W) { return W == 128 || W == 256 || W == 512 || W == 768; }

int mlp_bm(int mode, int W) { return (W <= 256 && mlp_occupancy(mode, W) == 1) ? 128 : 64; }

bool mlp_pairs_positions(int mode, int W) { return mode != MLP_ROUTED && mlp_waves(mode, W) == 8; }

int mlp_workgroups_per_cu(int mode, int W) { return mlp_occupancy(mode, W); }

bool mlp_mx_supported(int mode, int W) {
  return W == 512 || (W == 256 && mode == MLP_DENSE) || (W == 768 && mode != MLP_DENSE);
}

namespace {
template <int W, int MODE>
void launch_mx_wm(const MlpArgs& a, int grid, hipStream_t s) {
  constexpr int NW = mlp_waves(MODE, W), OCC = mlp_occupancy(MODE, W);
  static_assert(NW == 4, "the MXFP8 kernels are the 4-wave kernels");
  // (the Mix sub-layer reads its residual again: with the raw rows kept in
  // registers as in the bf16 kernel, the W = 256 MXFP8 main loop would spill)
  if (MODE != MLP_ROUTED && a.extra)
    hipLaunchKernelGGL((mlp_kernel<W, MODE, NW, OCC, MODE != MLP_ROUTED ? RV_EXTRA : RV_PLAIN, true>), dim3(grid),
                       dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_kernel<W, MODE, NW, OCC, RV_PLAIN, true>), dim3(grid), dim3(64 * NW), 0, s, a);
}
}  // namespace

hipError_t launch_mlp_mx(int mode, int W, const MlpArgs& a, int tiles, int workers, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  if (!mlp_mx_supported(mode, W) || a.hidden % MLP_HC != 0 || a.hidden > mx_max_chunks(W) * MLP_HC ||
      a.wrec < mx_rec_dwords(W, a.hidden) || a.wrec % 4 != 0)
    return hipErrorInvalidValue;
  workers = (workers & ~7) * mlp_workgroups_per_cu(mode, W);
  const int grid = (workers <= 0 || tiles <= workers) ? tiles : workers;
  if (W == 256) {
    launch_mx_wm<256, MLP_DENSE>(a, grid, s);
  } else if (W == 768) {
    if (mode == MLP_ROUTED) launch_mx_wm<768, MLP_ROUTED>(a, grid, s);
    else launch_mx_wm<768, MLP_SHARED>(a, grid, s);
  } else {
    switch (mode) {
      case MLP_DENSE: launch_mx_wm<512, MLP_DENSE>(a, grid, s); break;
      case MLP_ROUTED: launch_mx_wm<512, MLP_ROUTED>(a, grid, s); break;
      default: launch_mx_wm<512, MLP_SHARED>(a, grid, s); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_mlp(int mode, int W, const MlpArgs& a, int tiles, int workers, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  // persistent grid: at most `workers` workgroups per CU round, a multiple
  // of 8 so that a workgroup's tiles all sit on its own XCD
  workers = (workers & ~7) * mlp_workgroups_per_cu(mode, W);
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
