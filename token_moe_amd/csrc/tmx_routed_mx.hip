// tmx_routed_mx.hip -- the grouped routed-expert MLP of the Sparse-Pertoken
// MoE (TokenMixer-Large summary Eq. 19, section 2.5.1 MoEGroupedSwiGLU) for
// wide rows (W = 768, h_e = 384) with MXFP8 GEMM operands (section 2.5.2,
// FP8 E4M3 serving): E4M3 elements with one power-of-two (E8M0) scale per 32
// values along each GEMM's contraction axis, on gfx950's scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The tile is the 128-row tile of the bf16 routed kernel (tmx_routed.hip):
// 128 rows of one (position, expert) bucket, 4 waves, every weight fragment
// serving four 32-row MFMA blocks, in phases that each stay within the 256
// accumulator registers:
//
//   GEMM1 A  S_gate, S_up for hidden blocks 2w, 2w+1 of wave w, K-outer over
//            the 12 64-column slabs of the rows' x_hat (one MFMA k-step each)
//   U(A)     E4M3(silu(S_gate) * S_up) with one scale per row and 32 hidden
//            units -> LDS U [128, h_e]
//   GEMM1 B  hidden block 8 + w; U(B) -> LDS U
//   GEMM2 c  O [128, 256c : 256c + 256) = U @ W_down (2 column blocks per
//            wave), c = 0, 1, 2, each followed by gate * O -> bf16, staged in
//            LDS and written as whole 16-byte units.
//
// x_hat arrives quantised: the router writes an MXFP8 copy of its rows (E4M3
// codes and one exponent per 32 columns, the same quantisation as every
// other MXFP8 GEMM operand here), which this kernel gathers into an LDS copy
// of the whole tile (128 x 768 codes, 96 KiB) that both GEMM1 passes read:
// GEMM1 B runs from LDS alone. Slabs are copied into LDS 4 slabs ahead of
// the MFMAs that use them, during GEMM1 A (slabs 4..11) and the previous
// tile's GEMM2 parts (slabs 0..3); their global loads run 4 slabs ahead of
// the copy (four register sets of 32 bytes per lane). During the GEMM2
// parts, slabs 4..11 of the copy hold the epilogue's staging rows.
//
// The weights come from the MXFP8 packing of load time (launch_pack_mx):
// 2 KiB fragments, and per-lane scale records in the layout the fused MLP
// kernel reads them in (record wave = the fused kernel's owner of a column
// block); each wave reads the records of the blocks it computes, from global
// memory into registers, one phase ahead of their use. Weight fragments
// stream through a 12-slot register ring (24 KiB in flight per wave) in one
// order per tile (GEMM1 A, GEMM1 B, GEMM2 0, 1, 2) running on into the next
// tile.
#include <type_traits>

#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int RX_NT = 256;   // 4 waves
constexpr int RX_RB = 4;     // 32-row blocks per tile
constexpr int RX_BM = 32 * RX_RB;
constexpr int RX_SC = 64;    // columns per x_hat slab: one fp8 MFMA k-step
constexpr int RX_RING = 12;  // weight fragments in flight per wave
constexpr int RX_QA = 4;     // slabs between a slab's copy into LDS and its MFMAs
constexpr int RX_SETS = 4;   // register sets of slab loads in flight (slab s in set s % 4)
constexpr int RX_QMAX = 64;  // positions per tile queue whose tile counts sit in LDS
constexpr int RX_RSRC_W3 = 0x00020000;   // buffer resource word 3: raw 32-bit data, no swizzle

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 rx_join(const v4u& a, const v4u& b) {
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// scaled E4M3 MFMA: the A scale is byte OA of sa, the B scale byte 0 of sb;
// lane l supplies the scale of (row / column l % 32, K-block l / 32)
template <int OA>
__device__ __forceinline__ f32x16 rx_mfma(const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, (int)sa, 0, (int)sb);
}
__device__ __forceinline__ f32x16 rx_mfma_s(int oa, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb,
                                            const f32x16& c) {
  switch (oa) {
    case 0: return rx_mfma<0>(a, b, sa, sb, c);
    case 1: return rx_mfma<1>(a, b, sa, sb, c);
    case 2: return rx_mfma<2>(a, b, sa, sb, c);
    default: return rx_mfma<3>(a, b, sa, sb, c);
  }
}

// E4M3 bytes of x[0..3] * sc, clamped to +-448 first (the hardware
// conversion rounds to nearest even but does not saturate)
__device__ __forceinline__ uint32_t rx_e4m3x4(float x0, float x1, float x2, float x3, float sc) {
  x0 = fminf(fmaxf(x0 * sc, -448.f), 448.f);
  x1 = fminf(fmaxf(x1 * sc, -448.f), 448.f);
  x2 = fminf(fmaxf(x2 * sc, -448.f), 448.f);
  x3 = fminf(fmaxf(x3 * sc, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}
// shared exponent of a block with largest magnitude amax: floor(log2(amax))
// - 8 (E4M3's largest normal is 1.75 * 2^8), clamped to the E8M0 range
__device__ __forceinline__ int rx_exp(float amax) {
  int e = 0;
  (void)frexpf(amax, &e);
  const int k = amax > 0.f ? e - 9 : -127;
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

__device__ __forceinline__ float rx_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <int W, int HE>
struct RxShape {
  static constexpr int BM = RX_BM;
  static constexpr int HA = 2;                    // hidden blocks per wave, GEMM1 pass A
  static constexpr int HBB = HE / 128 - HA;       // ... pass B
  static constexpr int NSP = W / RX_SC;           // slabs (= k-steps) per GEMM1 pass
  static constexpr int KS = W / 64;               // k-steps of a gate / up fragment column
  static constexpr int KB2 = HE / 64;             // GEMM2 k-steps
  static constexpr int FA = 2 * HA, FB = 2 * HBB, FC = 2;     // fragments per k-step
  static constexpr int LA = NSP * FA, LB = NSP * FB, LC = KB2 * FC;   // fragments per phase
  static constexpr int USB = HE + 16;             // U row stride (bytes)
  static constexpr int USC = HE / 32;             // U scale bytes per row
  static constexpr int XSL = BM * RX_SC;          // code bytes per slab of the x_hat copy
  static constexpr int SU = BM * RX_SC / 16 / RX_NT;  // 16-byte code units of a slab per lane
  static constexpr int XE = W / 32;               // exponent bytes per x_hat row
  static constexpr int HS = 256 + 8;              // staged part-row stride (bf16)
  // LDS: x_hat codes [slab][row][64] (slabs RX_QA.. and a pad after them
  // double as the staging rows [128][HS]), x_hat exponents [row][XE],
  // U [row][USB], U exponents [row][hidden block]
  static constexpr int STG_PAD = BM * HS * 2 > (NSP - RX_QA) * XSL ? BM * HS * 2 - (NSP - RX_QA) * XSL : 0;
  static constexpr int OFF_XSC = NSP * XSL + STG_PAD;
  static constexpr int OFF_US = OFF_XSC + BM * XE;
  static constexpr int OFF_USC = OFF_US + BM * USB;
  static constexpr int LDS_BYTES = OFF_USC + BM * USC;
  static_assert(W == 768 && HE == 384, "the MXFP8 wide routed kernel is built for W 768, h_e 384");
  static_assert(HBB == 1 && NSP == 12 && SU == 2 && NSP - RX_QA == 2 * RX_SETS && XE % 4 == 0 &&
                BM * XE / 4 == 3 * RX_NT,
                "pass shapes: slab pipeline and exponent rows as laid out below");
  static_assert((W / 128) % 2 == 0, "GEMM2 scale byte: a down block's index among its record's blocks has j's parity");
  static_assert(LA % RX_RING == 0 && LB % RX_RING == 0 && LC % RX_RING == 0 && RX_RING % FA == 0 &&
                RX_RING % FB == 0 && RX_RING % FC == 0,
                "every phase is whole turns of the ring, each of whole k-steps");
  static_assert(LDS_BYTES + 3 * 2 * BM * 4 + 4 * (RX_QMAX + 2) <= 160 * 1024, "LDS budget");
};

template <int W, int HE>
__global__ __launch_bounds__(RX_NT, 1) void routed_mx_kernel(const MlpArgs a) {
  using S = RxShape<W, HE>;
  constexpr int BM = S::BM, HA = S::HA, HBB = S::HBB, NSP = S::NSP;
  constexpr int KS = S::KS, KB2 = S::KB2, FA = S::FA, FB = S::FB, FC = S::FC;
  constexpr int LA = S::LA, LB = S::LB, LC = S::LC, USB = S::USB, USC = S::USC, XSL = S::XSL, SU = S::SU;
  constexpr int HS = S::HS;
  constexpr int NBO = W / 128;   // the fused kernel's down column blocks per wave (record layout)

  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS_BYTES];
  __shared__ int rowb[2][BM];      // sample row of each tile row (-1: padding)
  __shared__ int rowgi[2][BM];     // expert-output row (b, p, slot)
  __shared__ float rowg[2][BM];    // gate of each tile row
  __shared__ int qcum[RX_QMAX + 1];   // tiles of the queue's positions before position q
  __shared__ int claim;
  uint8_t* const xq = lds;
  uint8_t* const xsc = lds + S::OFF_XSC;
  uint8_t* const us = lds + S::OFF_US;
  uint8_t* const usc = lds + S::OFF_USC;
  // staging rows of the GEMM2 epilogue, over slabs RX_QA.. of the x_hat copy
  // (free from the end of GEMM1 B to the next tile's GEMM1 A)
  uint16_t* const stg = reinterpret_cast<uint16_t*>(lds + RX_QA * XSL);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // lane-dependent addresses read `ot`, an opaque copy of the thread index
  // made anew before each phase (the compiler then does not hoist one
  // phase's addresses out of the tile loop)
  int ot = tid;
  auto fresh = [&]() __attribute__((always_inline)) { asm volatile("" : "+v"(ot)); };

  // ---- tile queues, as the bf16 routed kernel; the queue's tile counts are
  // read once into LDS as running sums, and a claim is decoded with one
  // ballot over them
  const bool split_q = (a.P & 7) == 0;
  const int qx = split_q ? (int)(blockIdx.x & 7) : 0;
  const int NPX = split_q ? (a.P >> 3) : a.P;
  const bool qlds = NPX <= RX_QMAX;
  if (qlds && tid < 64) {
    int n = tid < NPX ? a.ntiles[qx * NPX + tid] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(n, d, 64);
      if (lane >= d) n += v;
    }
    qcum[tid + 1] = n;
    if (tid == 0) qcum[0] = 0;
  }
  struct Tile {
    int p, group, start, nrows;
  };
  auto qdecode = [&](int k, Tile& T) -> bool {
    int p;
    if (qlds) {
      const bool hit = lane < NPX && qcum[lane] <= k && k < qcum[lane + 1];
      const uint64_t m = __ballot(hit);
      if (m == 0) return false;
      const int q = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
      p = qx * NPX + q;
      k -= qcum[q];
    } else {
      p = qx * NPX;
      int q = 0;
      for (; q < NPX; ++q, ++p) {
        const int n = a.ntiles[p];
        if (k < n) break;
        k -= n;
      }
      if (q == NPX) return false;
    }
    const int4 tl = a.tiles[(size_t)p * a.max_tiles + k];
    T.p = __builtin_amdgcn_readfirstlane(p);
    T.group = __builtin_amdgcn_readfirstlane(p * a.E + tl.x);
    T.start = __builtin_amdgcn_readfirstlane(tl.y);
    T.nrows = __builtin_amdgcn_readfirstlane(tl.z);
    return true;
  };
  auto set_rows = [&](const Tile& T, int buf) {
    for (int r = tid; r < BM; r += RX_NT) {
      int b = -1, gi = 0;
      float g = 0.f;
      if (r < T.nrows) {
        const int ent = a.rows[(size_t)T.p * a.B * a.top_k + T.start + r];   // b * top_k + slot
        b = ent / a.top_k;
        gi = (b * a.P + T.p) * a.top_k + (ent - b * a.top_k);
        g = a.gate[gi];
      }
      rowb[buf][r] = b;
      rowgi[buf][r] = gi;
      rowg[buf][r] = g;
    }
  };

  // ---- weight stream of a tile, phase by phase:
  //   0  GEMM1 A: k-step kb, hidden block HA wave + h, gate / up
  //   1  GEMM1 B: hidden block 4 HA + HBB wave
  //   2, 3, 4  GEMM2 part c = ph - 2: k-step kb, output block 8 c + 2 wave + j
  //   5  the next tile's phase 0
  // A super-step is one turn of the ring; slot i is refilled with fragment i
  // of the next super-step, which may belong to the next phase. Fragments
  // are 2 KiB (two 1 KiB halves, 16 bytes per lane each), read through
  // buffer resources with a 32-bit lane offset.
  constexpr uint32_t GU_BYTES = 2u * W * HE;        // gate|up codes of a bucket
  constexpr uint32_t WD_BYTES = (uint32_t)HE * W;   // down codes of a bucket
  auto rsrc = [](const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RX_RSRC_W3);
  };
  const uint8_t* const wgu8 = reinterpret_cast<const uint8_t*>(a.wgu);
  const uint8_t* const wd8 = reinterpret_cast<const uint8_t*>(a.wd);
  __amdgpu_buffer_rsrc_t cgu, cwd, ngu, nwd;
  auto bases = [&](const Tile& T, __amdgpu_buffer_rsrc_t& gu, __amdgpu_buffer_rsrc_t& wd) {
    gu = rsrc(wgu8 + (size_t)T.group * GU_BYTES, GU_BYTES);
    wd = rsrc(wd8 + (size_t)T.group * WD_BYTES, WD_BYTES);
  };
  // the fragment's constant offset is added to `zs`, an opaque zero made
  // anew for every k-step: the compiler would otherwise hoist the ~100
  // constant offsets of a tile out of the tile loop into scalar registers,
  // which then spill
  int zs = 0;
  auto frag = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, int c) __attribute__((always_inline)) -> i32x8 {
    return rx_join(__builtin_amdgcn_raw_buffer_load_b128(r, voff + 0u, zs + c, 0),
                   __builtin_amdgcn_raw_buffer_load_b128(r, voff + 1024u, zs + c, 0));
  };
  // gate / up fragment (block nb, k-step kb, which) at byte ((nb KS + kb) 2 +
  // which) 2048; down fragment (k-step kb, block ob) at (kb W/32 + ob) 2048
  auto wload = [&](int ph, int pos) __attribute__((always_inline)) -> i32x8 {
    const uint32_t lo = (uint32_t)(ot & 63) * 16u;
    if (ph == 0 || ph == 5) {
      const int kb = pos / FA, ii = pos % FA;
      const int nb = HA * wave + (ii >> 1);
      return frag(ph == 0 ? cgu : ngu, lo, ((nb * KS + kb) * 2 + (ii & 1)) * 2048);
    }
    if (ph == 1) {
      const int kb = pos / FB, ii = pos % FB;
      const int nb = 4 * HA + HBB * wave + (ii >> 1);
      return frag(cgu, lo, ((nb * KS + kb) * 2 + (ii & 1)) * 2048);
    }
    const int kb = pos / FC, j = pos % FC;
    const int ob = 8 * (ph - 2) + 2 * wave + j;
    return frag(cwd, lo, (kb * (W / 32) + ob) * 2048);
  };
  constexpr int SA = LA / RX_RING, SB = LB / RX_RING, SCC = LC / RX_RING;   // super-steps per phase
  auto refill = [&](i32x8& dst, auto ph_tag, int i, int sn) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_tag)::value;
    constexpr int NSS = PH == 0 ? SA : PH == 1 ? SB : SCC;
    dst = sn < NSS ? wload(PH, sn * RX_RING + i) : wload(PH + 1, (sn - NSS) * RX_RING + i);
  };
  i32x8 ring[RX_RING];

  // ---- weight scales: dword q of matrix m (0 gate, 1 up, 2 down) of hidden
  // chunk c in the record of (group, record wave rw) and this lane
  constexpr int DW = W / 256;
  auto rec_dw = [&](const Tile& T, int rw, int c, int m, int q) __attribute__((always_inline)) -> uint32_t {
    return a.wsc[(((size_t)T.group * 4 + rw) * 64 + lane) * a.wrec + (c * 3 + m) * DW + q];
  };
  // GEMM1 pass scales: [block h][gate, up][dword of 4 k-steps]
  struct ScA {
    uint32_t w[HA][2][DW];
  };
  struct ScB {
    uint32_t w[HBB][2][DW];
  };
  // GEMM2 part scales: [block j][hidden chunk]: byte 2 (jj % 2) + t of the
  // dword, jj = the block's index among its record wave's NBO blocks
  struct ScC {
    uint32_t w[FC][HE / 128];
  };
  auto load_sa = [&](const Tile& T, ScA& s) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < HA; ++h) {
      const int nb = HA * wave + h;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < DW; ++q) s.w[h][m][q] = rec_dw(T, nb % 4, nb / 4, m, q);
    }
  };
  auto load_sb = [&](const Tile& T, ScB& s) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < HBB; ++h) {
      const int nb = 4 * HA + HBB * wave + h;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < DW; ++q) s.w[h][m][q] = rec_dw(T, nb % 4, nb / 4, m, q);
    }
  };
  auto load_sc = [&](const Tile& T, int part, ScC& s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FC; ++j) {
      const int ob = 8 * part + 2 * wave + j, jj = ob % NBO;
#pragma unroll
      for (int c = 0; c < HE / 128; ++c) s.w[j][c] = rec_dw(T, ob / NBO, c, 2, (2 * jj) >> 2);
    }
  };

  // ---- x_hat slabs, from the router's MXFP8 copy of x_hat (E4M3 codes
  // [P][B][W], exponents [P][B][W/32]): unit u = tid + 256 i of a slab is row
  // u / 4, 16-column chunk u % 4 of the slab's 64 columns. In LDS a row's
  // chunk k sits at chunk k ^ (row % 4) (the fragment reads of 4 consecutive
  // rows hit different bank groups); the tile's exponents are copied whole,
  // [row][W/32].
  // byte offsets of this lane's slab units in the codes, for this tile
  // (roff) and the next (roffn; rows of padding read sample row 0)
  uint32_t roff[SU], roffn[SU];
  auto slab_rows = [&](int p, int tb, uint32_t* ro) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RX_NT;
      const int b = rowb[tb][u >> 2];
      ro[i] = ((uint32_t)p * (uint32_t)a.B + (uint32_t)(b < 0 ? 0 : b)) * (uint32_t)W + (uint32_t)(u & 3) * 16u;
    }
  };
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.xq8, (uint32_t)((uint64_t)a.P * a.B * W));
  const __amdgpu_buffer_rsrc_t er = rsrc(a.xe8, (uint32_t)((uint64_t)a.P * a.B * S::XE));
  // slab s of this tile (nxt: of the next tile)
  auto slab_load = [&](int s, bool nxt, v4u* v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SU; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, nxt ? roffn[i] : roff[i], s * RX_SC, 0);
  };
  auto slab_store = [&](int s, const v4u* v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RX_NT, r = u >> 2;
      *reinterpret_cast<v4u*>(&xq[s * XSL + r * RX_SC + (((u & 3) ^ (r & 3)) * 16)]) = v[i];
    }
  };
  // the exponents of the tile at position p with row table tb: dword d =
  // tid + 256 j of the tile's [128][XE] bytes
  auto exp_load = [&](int p, int tb, uint32_t* e) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int d = ot + j * RX_NT, r = d / (S::XE / 4);
      const int b = rowb[tb][r];
      e[j] = __builtin_amdgcn_raw_buffer_load_b32(
          er, ((uint32_t)p * (uint32_t)a.B + (uint32_t)(b < 0 ? 0 : b)) * (uint32_t)S::XE, (d - r * (S::XE / 4)) * 4, 0);
    }
  };
  auto exp_store = [&](const uint32_t* e) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 3; ++j) reinterpret_cast<uint32_t*>(xsc)[ot + j * RX_NT] = e[j];
  };
  // B operand of row block rb from slab s: row 32 rb + l32, bytes 16 h32 ..
  // of K-block 0 and 32 + 16 h32 .. of K-block 1; its exponent in byte 0
  auto x_frag = [&](int s, int rb) -> i32x8 {
    const int r = rb * 32 + (ot & 31), h = (ot >> 5) & 1;
    const uint8_t* row = xq + s * XSL + r * RX_SC;
    return rx_join(*reinterpret_cast<const v4u*>(row + ((h ^ (r & 3)) * 16)),
                   *reinterpret_cast<const v4u*>(row + (((2 + h) ^ (r & 3)) * 16)));
  };
  auto x_scale = [&](int s, int rb) -> uint32_t {
    const int r = rb * 32 + (ot & 31), h = (ot >> 5) & 1;
    return (uint32_t)xsc[r * S::XE + 2 * s + h];
  };
  // B operand of GEMM2 k-step kb: U row 32 rb + l32, hidden 64 kb + 16 h32 ..
  // (K-block 0) and 64 kb + 32 + 16 h32 .. (K-block 1); scale of hidden block
  // 2 kb + h32 in byte 0
  auto u_frag = [&](int rb, int kb) -> i32x8 {
    const uint8_t* row = us + (rb * 32 + (ot & 31)) * USB + kb * 64 + ((ot >> 5) & 1) * 16;
    return rx_join(*reinterpret_cast<const v4u*>(row), *reinterpret_cast<const v4u*>(row + 32));
  };
  auto u_scale = [&](int rb, int kb) -> uint32_t {
    return (uint32_t)usc[(rb * 32 + (ot & 31)) * USC + 2 * kb + ((ot >> 5) & 1)];
  };

  // ---- first tile: slabs 0..3 and the exponents in LDS, 4..7 loading ---------
  Tile cur, nx;
  if (tid == 0) claim = atomicAdd(&a.qhead[qx], 1);
  __syncthreads();   // also publishes qcum
  if (!qdecode(claim, cur)) return;                  // uniform per workgroup
  __syncthreads();
  if (tid == 0) claim = atomicAdd(&a.qhead[qx], 1);
  __syncthreads();
  bool has_nx = qdecode(claim, nx);
  if (!has_nx) nx = cur;
  set_rows(cur, 0);
  set_rows(nx, 1);
  bases(cur, cgu, cwd);
  bases(nx, ngu, nwd);
  __syncthreads();
  int buf = 0;
  v4u sv[RX_SETS][SU];   // slab s waits in register set s % 4
  slab_rows(cur.p, 0, roff);
  slab_rows(nx.p, 1, roffn);
  ScA sa;
  {
    uint32_t e[3];
#pragma unroll
    for (int k = 0; k < RX_SETS; ++k) slab_load(k, false, sv[k]);
    exp_load(cur.p, 0, e);
    load_sa(cur, sa);
#pragma unroll
    for (int f = 0; f < RX_RING; ++f) ring[f] = wload(0, f);
#pragma unroll
    for (int k = 0; k < RX_SETS; ++k) {
      slab_store(k, sv[k]);
      slab_load(k + RX_SETS, false, sv[k]);
    }
    exp_store(e);
  }
  __syncthreads();

  while (true) {
    fresh();
    i32x8 xb[RX_RB];
    uint32_t xs[RX_RB];
#pragma unroll
    for (int rb = 0; rb < RX_RB; ++rb) {
      xb[rb] = x_frag(0, rb);
      xs[rb] = x_scale(0, rb);
    }
    ScB sbs;

    // ---- GEMM1 k-step t of pass PH (slab t; t compile-time). Pass A also
    // copies slab t + 4 from register set t % 4 into LDS, and that set then
    // loads slab t + 8 (past slab 11: the next tile's slab t - 4). A barrier
    // after k-steps 2, 5 and 7 publishes the slabs copied since the previous
    // one, each read (as the operand of the k-step before its own) at least
    // one k-step later. The row blocks' x_hat operands are replaced by the
    // next slab's as soon as their MFMAs have issued.
    auto kstep = [&](auto ph_tag, auto t_tag, auto& sg, auto& su, const auto& sc) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value, t = decltype(t_tag)::value;
      constexpr int F = PH == 0 ? FA : FB;
      constexpr bool COPY = PH == 0 && t + RX_QA < NSP;
      constexpr int QS = t % RX_SETS;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb) {
#pragma unroll
        for (int i = 0; i < F; ++i) {
          // the pass's first k-step takes a zero accumulator operand
          f32x16& acc = (i & 1) ? su[rb][i >> 1] : sg[rb][i >> 1];
          acc = rx_mfma_s(t & 3, ring[(t * F + i) % RX_RING], xb[rb], sc.w[i >> 1][i & 1][t >> 2], xs[rb],
                          t == 0 ? f32x16{} : acc);
        }
        if (t + 1 < NSP) {
          xb[rb] = x_frag(t + 1, rb);
          xs[rb] = x_scale(t + 1, rb);
        }
      }
      asm volatile("" : "+s"(zs));
      if (COPY) {
        slab_store(t + RX_QA, sv[QS]);
        if (t + 2 * RX_SETS < NSP)
          slab_load(t + 2 * RX_SETS, false, sv[QS]);
        else
          slab_load(t + 2 * RX_SETS - NSP, true, sv[QS]);
      }
      // GEMM1 B's scales
      if (PH == 0 && t == NSP - RX_QA) load_sb(cur, sbs);
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int pos = t * F + i;
        refill(ring[pos % RX_RING], std::integral_constant<int, PH>{}, pos % RX_RING, pos / RX_RING + 1);
      }
      // the k-step's products are taken here: the compiler would otherwise
      // sink the MFMAs (pure operations) down to the accumulators' use after
      // the pass, keeping every k-step's operands live until then
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb)
#pragma unroll
        for (int h = 0; h < F / 2; ++h) asm volatile("" : "+a"(sg[rb][h]), "+a"(su[rb][h]));
      if (PH == 0 && (t == 2 || t == 5 || t == NSP - RX_QA - 1)) __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // U of a pass's hidden blocks (block nb0 + h of the wave) -> LDS: one
    // scale per row and block (16 values in this lane, 16 in lane ^ 32)
    auto store_u = [&](int nb0, auto& sg, auto& su, auto nh_tag) __attribute__((always_inline)) {
      constexpr int NH = decltype(nh_tag)::value;
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          float u[16], am = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            u[e] = rx_silu(sg[rb][h][e]) * su[rb][h][e];
            am = fmaxf(am, fabsf(u[e]));
          }
          am = fmaxf(am, __shfl_xor(am, 32, 64));
          const int k = rx_exp(am);
          const float sc = ldexpf(1.f, -k);
          const int row = rb * 32 + (ot & 31), nb = nb0 + h;
          uint8_t* dst = us + row * USB + nb * 32 + 4 * ((ot >> 5) & 1);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<uint32_t*>(dst + 8 * g4) = rx_e4m3x4(u[4 * g4], u[4 * g4 + 1], u[4 * g4 + 2],
                                                                    u[4 * g4 + 3], sc);
          usc[row * USC + nb] = (uint8_t)(k + 127);   // lanes l and l ^ 32 store the same byte
          // one accumulator block at a time: the scheduler would otherwise
          // move every accumulator to VGPRs at once
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto pass = [&](auto ph_tag, auto& sg, auto& su, const auto& sc) __attribute__((always_inline)) {
      kstep(ph_tag, std::integral_constant<int, 0>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 1>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 2>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 3>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 4>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 5>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 6>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 7>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 8>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 9>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 10>{}, sg, su, sc);
      kstep(ph_tag, std::integral_constant<int, 11>{}, sg, su, sc);
    };

    // ================= GEMM1 pass A =================
    {
      f32x16 sg[RX_RB][HA], su[RX_RB][HA];
      pass(std::integral_constant<int, 0>{}, sg, su, sa);
      // pass B starts on slab 0 again
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb) {
        xb[rb] = x_frag(0, rb);
        xs[rb] = x_scale(0, rb);
      }
      store_u(HA * wave, sg, su, std::integral_constant<int, HA>{});
    }
    ScC scc;
    load_sc(cur, 0, scc);
    // ================= GEMM1 pass B (x_hat from LDS only) =================
    fresh();
    {
      f32x16 sg[RX_RB][HBB], su[RX_RB][HBB];
      pass(std::integral_constant<int, 1>{}, sg, su, sbs);
      store_u(4 * HA + HBB * wave, sg, su, std::integral_constant<int, HBB>{});
    }
    __syncthreads();   // U complete; every wave is done with the x_hat copy

    // the claim of the tile after next goes out now (read after the epilogue)
    int qnext = 0;
    if (tid == 0) qnext = atomicAdd(&a.qhead[qx], 1);

    // ================= GEMM2 parts, each with its epilogue =================
    uint32_t en[3];   // the next tile's exponents, from part 1 to part 2
    // The parts also quantise the next tile's slabs 0..3 into the x_hat copy
    // (one unit per k-step; part 0 takes slabs 0 and 1), each register set
    // then loading the next tile's slab two further on.
    auto gemm2_part = [&](auto ph_tag, f32x16 (&o)[RX_RB][FC], const ScC& s) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value, C = PH - 2;
      i32x8 ub[RX_RB];
      uint32_t uss[RX_RB];
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb) {
        ub[rb] = u_frag(rb, 0);
        uss[rb] = u_scale(rb, 0);
      }
#pragma unroll
      for (int kb = 0; kb < KB2; ++kb) {
        __builtin_amdgcn_sched_barrier(0);
        // past the last k-step the prefetch reads k-step 0 again (unused)
        const int kn = kb + 1 < KB2 ? kb + 1 : 0;
#pragma unroll
        for (int rb = 0; rb < RX_RB; ++rb) {
#pragma unroll
          for (int j = 0; j < FC; ++j) {
            // byte 2 (jj % 2) + kb % 2 of the chunk's dword, jj = ob % NBO:
            // ob = 8 part + 2 wave + j and NBO is even, so jj % 2 = j
            o[rb][j] = rx_mfma_s(2 * j + (kb & 1), ring[(kb * FC + j) % RX_RING], ub[rb], s.w[j][kb >> 1], uss[rb],
                                 kb == 0 ? f32x16{} : o[rb][j]);
          }
          ub[rb] = u_frag(rb, kn);
          uss[rb] = u_scale(rb, kn);
        }
        // the next tile: parts 0 and 1 copy its slabs 2C, 2C + 1 into LDS
        // (k-steps 1, 3), their register sets then loading slabs 2C + 4,
        // 2C + 5; part 1 loads its exponents (k-step 0), part 2 stores them
        asm volatile("" : "+s"(zs));
        if (C < 2 && (kb == 1 || kb == 3)) {
          const int sl = 2 * C + (kb >> 1);
          slab_store(sl, sv[sl]);
          slab_load(sl + RX_SETS, true, sv[sl]);
        }
        if (C == 1 && kb == 0) exp_load(nx.p, buf ^ 1, en);
        if (C == 2 && kb == 0) exp_store(en);
#pragma unroll
        for (int j = 0; j < FC; ++j) {
          const int pos = kb * FC + j;
          refill(ring[pos % RX_RING], std::integral_constant<int, PH>{}, pos % RX_RING, pos / RX_RING + 1);
        }
        // the k-step's products are taken here (as in GEMM1)
#pragma unroll
        for (int rb = 0; rb < RX_RB; ++rb)
#pragma unroll
          for (int j = 0; j < FC; ++j) asm volatile("" : "+a"(o[rb][j]));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // gate * O of row block rb -> staging rows
    auto stage_rb = [&](int rb, f32x16 (&o)[RX_RB][FC]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < FC; ++j) asm volatile("" : "+a"(o[rb][j]));
      const int row = rb * 32 + (ot & 31);
      const float g = rowg[buf][row];
#pragma unroll
      for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 w2;
          w2.x = pack_bf16x2(g * o[rb][j][4 * g4], g * o[rb][j][4 * g4 + 1]);
          w2.y = pack_bf16x2(g * o[rb][j][4 * g4 + 2], g * o[rb][j][4 * g4 + 3]);
          *reinterpret_cast<uint2*>(&stg[row * HS + (2 * wave + j) * 32 + 8 * g4 + 4 * ((ot >> 5) & 1)]) = w2;
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    // staged rows [row0, row0 + 32) of part c -> the expert-output rows (32
    // 16-byte units per part row; the batch's LDS reads go out before its
    // stores)
    auto store_rows = [&](int row0, int c) __attribute__((always_inline)) {
      constexpr int U8P = 256 / 8, NU = 32 * U8P / RX_NT;
      v4u v[NU];
      int gi[NU], c8s[NU];
      bool ok[NU];
#pragma unroll
      for (int k = 0; k < NU; ++k) {
        const int u = ot + k * RX_NT, r = u / U8P, c8 = u - r * U8P, row = row0 + r;
        v[k] = *reinterpret_cast<const v4u*>(&stg[row * HS + c8 * 8]);
        ok[k] = rowb[buf][row] >= 0;
        gi[k] = rowgi[buf][row];
        c8s[k] = c8;
      }
#pragma unroll
      for (int k = 0; k < NU; ++k)
        if (ok[k])
          __builtin_nontemporal_store(v[k], reinterpret_cast<v4u*>(a.part + (size_t)gi[k] * W + c * 256 + c8s[k] * 8));
    };
    auto part = [&](auto ph_tag, const ScC& s) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value;
      fresh();
      f32x16 o[RX_RB][FC];
      gemm2_part(ph_tag, o, s);
      fresh();
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb) stage_rb(rb, o);
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb) store_rows(rb * 32, PH - 2);
      __syncthreads();
    };
    {
      ScC s1;
      load_sc(cur, 1, s1);
      part(std::integral_constant<int, 2>{}, scc);
      ScC s2;
      load_sc(cur, 2, s2);
      part(std::integral_constant<int, 3>{}, s1);
      // the next tile's pass A scales (after the last tile: this tile's,
      // unused -- loads on one path only drain every load in flight)
      load_sa(has_nx ? nx : cur, sa);
      if (tid == 0) claim = qnext;
      part(std::integral_constant<int, 4>{}, s2);
    }
    if (!has_nx) break;

    // ---- the next tile; the one after it is decoded into the freed row table
    cur = nx;
    buf ^= 1;
    cgu = ngu;
    cwd = nwd;
#pragma unroll
    for (int i = 0; i < SU; ++i) roff[i] = roffn[i];
    has_nx = qdecode(claim, nx);
    if (!has_nx) nx = cur;
    set_rows(nx, buf ^ 1);
    bases(nx, ngu, nwd);
    __syncthreads();
    slab_rows(nx.p, buf ^ 1, roffn);
  }
}

}  // namespace

int routed_wide_mx_rows(int W, int h_e) { return (W == 768 && h_e == 384) ? RX_BM : 0; }

hipError_t launch_routed_wide_mx(const MlpArgs& a, int tiles, int workers, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  if (a.hidden != 384 || a.wrec < mx_rec_dwords(768, 384) || !a.xq8 || !a.xe8) return hipErrorInvalidValue;
  workers &= ~7;
  const int grid = (workers <= 0 || tiles <= workers) ? tiles : workers;
  hipLaunchKernelGGL((routed_mx_kernel<768, 384>), dim3(grid), dim3(RX_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tmx
