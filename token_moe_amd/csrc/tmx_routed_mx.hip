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
//   GEMM1 A  S_gate, S_up for hidden blocks 2w, 2w+1 of wave w, K-outer: the
//            rows' x_hat columns stream through LDS in 64-column slabs
//            (one MFMA k-step each), quantised to E4M3 as they are stored;
//   U(A)     E4M3(silu(S_gate) * S_up) with one scale per row and 32 hidden
//            units -> LDS U [128, h_e];
//   GEMM1 B  hidden block 8 + w, x_hat streamed again; U(B) -> LDS U;
//   GEMM2 c  O [128, 256c : 256c + 256) = U @ W_down (2 column blocks per
//            wave), c = 0, 1, 2, each followed by gate * O -> bf16, staged 32
//            rows at a time and written as whole 16-byte units.
//
// The weights come from the MXFP8 packing of load time (launch_pack_mx):
// 2 KiB fragments, and per-lane scale records in the layout the fused MLP
// kernel reads them in (record wave = the fused kernel's owner of a column
// block); each wave here reads the records of the blocks it computes, from
// global memory into registers, one phase ahead of their use.
//
// Pipelines as in the bf16 kernel: weight fragments stream through a
// 12-slot register ring (2 KiB fragments, 24 KiB in flight per wave) in one
// order per tile (GEMM1 A, GEMM1 B, GEMM2 0, 1, 2) running on into the next
// tile; x_hat slabs run through three LDS buffers, slab t + 1 quantised
// into its buffer and slab t + 3 loaded at slab step t.
#include <type_traits>

#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int RX_NT = 256;   // 4 waves
constexpr int RX_RB = 4;     // 32-row blocks per tile
constexpr int RX_BM = 32 * RX_RB;
constexpr int RX_SC = 64;    // columns per x_hat slab: one fp8 MFMA k-step
constexpr int RX_RING = 12;  // weight fragments in flight per wave
constexpr int RX_RSRC_W3 = 0x00020000;   // buffer resource word 3: raw 32-bit data, no swizzle
constexpr int RX_NT_POLICY = 2;          // streaming cache policy (the rows' last read)

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
  static constexpr int NP2 = W / 256;             // GEMM2 parts (2 output blocks per wave each)
  static constexpr int NSP = W / RX_SC;           // slabs (= k-steps) per GEMM1 pass
  static constexpr int NSL = 2 * NSP;             // slab steps per tile
  static constexpr int KS = W / 64;               // k-steps of a gate / up fragment column
  static constexpr int KB2 = HE / 64;             // GEMM2 k-steps
  static constexpr int FA = 2 * HA, FB = 2 * HBB, FC = 2;     // fragments per k-step
  static constexpr int LA = NSP * FA, LB = NSP * FB, LC = KB2 * FC;   // fragments per phase
  static constexpr int USB = HE + 16;             // U row stride (bytes)
  static constexpr int USC = HE / 32;             // U scale bytes per row
  static constexpr int SLAB = BM * RX_SC;         // code bytes per slab buffer
  static constexpr int SU = BM * RX_SC / 8 / RX_NT;   // 16-byte bf16 units of a slab per lane
  static constexpr int HS = 256 + 8;              // staged part-row stride (bf16)
  static constexpr int NR = HE / 32;              // hidden blocks (record scale bytes per row of U)
  static_assert(W == 768 && HE == 384, "the MXFP8 wide routed kernel is built for W 768, h_e 384");
  static_assert(HBB == 1 && NSP % 6 == 0, "pass shapes");
  static_assert((W / 128) % 2 == 0, "GEMM2 scale byte: a down block's index among its record's blocks has j's parity");
  static_assert(LA % RX_RING == 0 && LB % RX_RING == 0 && LC % RX_RING == 0 && RX_RING % FA == 0 &&
                RX_RING % FB == 0 && RX_RING % FC == 0,
                "every phase is whole turns of the ring, each of whole k-steps");
  static_assert(3 * (SLAB + 2 * BM) + BM * USB + BM * USC + 32 * HS * 2 + 3 * 2 * BM * 4 + 16 <= 160 * 1024,
                "LDS budget");
};

template <int W, int HE>
__global__ __launch_bounds__(RX_NT, 1) void routed_mx_kernel(const MlpArgs a) {
  using S = RxShape<W, HE>;
  constexpr int BM = S::BM, HA = S::HA, HBB = S::HBB, NP2 = S::NP2, NSP = S::NSP, NSL = S::NSL;
  constexpr int KS = S::KS, KB2 = S::KB2, FA = S::FA, FB = S::FB, FC = S::FC;
  constexpr int LA = S::LA, LB = S::LB, LC = S::LC, USB = S::USB, USC = S::USC, SLAB = S::SLAB, SU = S::SU;
  constexpr int HS = S::HS;
  constexpr int NBO = W / 128;   // the fused kernel's down column blocks per wave (record layout)

  __shared__ __attribute__((aligned(16))) uint8_t slabs[3 * SLAB];
  __shared__ __attribute__((aligned(16))) uint8_t slabsc[3 * 2 * BM];   // [buffer][row][2 K-blocks]
  __shared__ __attribute__((aligned(16))) uint8_t us[BM * USB];
  __shared__ __attribute__((aligned(16))) uint8_t usc[BM * USC];         // [row][hidden block]
  __shared__ __attribute__((aligned(16))) uint16_t stg[32 * HS];
  __shared__ int rowb[2][BM];      // sample row of each tile row (-1: padding)
  __shared__ int rowgi[2][BM];     // expert-output row (b, p, slot)
  __shared__ float rowg[2][BM];    // gate of each tile row
  __shared__ int claim;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // lane-dependent addresses read `ot`, an opaque copy of the thread index
  // made anew before each phase (the compiler then does not hoist one
  // phase's addresses out of the tile loop)
  int ot = tid;
  auto fresh = [&]() __attribute__((always_inline)) { asm volatile("" : "+v"(ot)); };

  // ---- tile queues, as the bf16 routed kernel
  const bool split_q = (a.P & 7) == 0;
  const int qx = split_q ? (int)(blockIdx.x & 7) : 0;
  const int NPX = split_q ? (a.P >> 3) : a.P;
  struct Tile {
    int p, group, start, nrows;
  };
  auto qdecode = [&](int k, Tile& T) -> bool {
    int p = qx * NPX;
    for (int q = 0; q < NPX; ++q, ++p) {
      const int n = a.ntiles[p];
      if (k < n) {
        const int4 tl = a.tiles[(size_t)p * a.max_tiles + k];
        T.p = __builtin_amdgcn_readfirstlane(p);
        T.group = __builtin_amdgcn_readfirstlane(p * a.E + tl.x);
        T.start = __builtin_amdgcn_readfirstlane(tl.y);
        T.nrows = __builtin_amdgcn_readfirstlane(tl.z);
        return true;
      }
      k -= n;
    }
    return false;
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
  // of the next super-step, which may belong to the next phase (both
  // addresses are formed and one selected: one unconditional load pair).
  // Fragment sizes are 2 KiB (two 1 KiB halves, 16 bytes per lane each),
  // read through buffer resources with a 32-bit lane offset.
  constexpr uint32_t GU_BYTES = 2u * W * HE;   // gate|up codes of a bucket
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
  auto frag = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, int c) __attribute__((always_inline)) -> i32x8 {
    return rx_join(__builtin_amdgcn_raw_buffer_load_b128(r, voff, c, 0),
                   __builtin_amdgcn_raw_buffer_load_b128(r, voff, c + 1024, 0));
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

  // ---- x_hat slabs: unit u = tid + 256 i of a slab is row u / 8, 8-column
  // chunk u % 8 of the slab's 64 columns (bf16 in memory). The slab is stored
  // quantised: 64 code bytes per row, 16-byte chunk k of a row at chunk k ^
  // (row % 4) (the fragment reads of 4 consecutive rows hit different bank
  // groups), and the row's two 32-column block exponents.
  uint32_t roff[SU], roffn[SU];
  auto slab_rows = [&](int p, int buf, uint32_t* ro) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RX_NT;
      const int b = rowb[buf][u >> 3];
      ro[i] = (((uint32_t)p * (uint32_t)a.B + (uint32_t)(b < 0 ? 0 : b)) * (uint32_t)W + (uint32_t)(u & 7) * 8u) * 2u;
    }
  };
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.xhat, (uint32_t)((uint64_t)a.P * a.B * W * 2));
  auto slab_load = [&](int t, v4u* v) __attribute__((always_inline)) {
    const bool nxt = t >= NSL;
    const int col = (nxt ? t - NSL : (t >= NSP ? t - NSP : t)) * RX_SC * 2;
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const uint32_t o = nxt ? roffn[i] : roff[i];
      v[i] = (t >= NSP && !nxt) ? __builtin_amdgcn_raw_buffer_load_b128(xr, o, col, RX_NT_POLICY)
                                : __builtin_amdgcn_raw_buffer_load_b128(xr, o, col, 0);
    }
  };
  // quantise and store: the 4 units of a 32-column block are 4 consecutive
  // lanes (u % 8 = 4k .. 4k + 3 of one row)
  auto slab_store = [&](int sb, const v4u* v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RX_NT, r = u >> 3, c8 = u & 7;
      const uint16_t* h = reinterpret_cast<const uint16_t*>(&v[i]);
      float n[8], am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        n[e] = bf2f(h[e]);
        am = fmaxf(am, fabsf(n[e]));
      }
      am = fmaxf(am, __shfl_xor(am, 1, 64));
      am = fmaxf(am, __shfl_xor(am, 2, 64));
      const int k = rx_exp(am);
      const float sc = ldexpf(1.f, -k);
      uint2 q;
      q.x = rx_e4m3x4(n[0], n[1], n[2], n[3], sc);
      q.y = rx_e4m3x4(n[4], n[5], n[6], n[7], sc);
      *reinterpret_cast<uint2*>(&slabs[sb * SLAB + r * RX_SC + (((c8 >> 1) ^ (r & 3)) * 16) + (c8 & 1) * 8]) = q;
      if ((c8 & 3) == 0) slabsc[(sb * BM + r) * 2 + (c8 >> 2)] = (uint8_t)(k + 127);
    }
  };
  // B operand of row block rb from a slab: row 32 rb + l32, bytes 16 h32 ..
  // of K-block 0 and 32 + 16 h32 .. of K-block 1; its scale in byte 0
  auto slab_frag = [&](int sb, int rb) -> i32x8 {
    const int r = rb * 32 + (ot & 31), h = (ot >> 5) & 1;
    const uint8_t* row = slabs + sb * SLAB + r * RX_SC;
    return rx_join(*reinterpret_cast<const v4u*>(row + ((h ^ (r & 3)) * 16)),
                   *reinterpret_cast<const v4u*>(row + (((2 + h) ^ (r & 3)) * 16)));
  };
  auto slab_scale = [&](int sb, int rb) -> uint32_t {
    const int r = rb * 32 + (ot & 31), h = (ot >> 5) & 1;
    return (uint32_t)slabsc[(sb * BM + r) * 2 + h];
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

  // ---- first tile -----------------------------------------------------------------
  Tile cur, nx;
  if (tid == 0) claim = atomicAdd(&a.qhead[qx], 1);
  __syncthreads();
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
  v4u sv[2][SU];   // slab t waits in register set t % 2
  slab_rows(cur.p, 0, roff);
  slab_rows(nx.p, 1, roffn);
  ScA sa;
  {
    v4u s0[SU];
    slab_load(0, s0);
    slab_load(1, sv[1]);
    slab_load(2, sv[0]);
    load_sa(cur, sa);
#pragma unroll
    for (int f = 0; f < RX_RING; ++f) ring[f] = wload(0, f);
    slab_store(0, s0);
  }
  __syncthreads();

  while (true) {
    fresh();
    i32x8 xb[RX_RB];
    uint32_t xs[RX_RB];
#pragma unroll
    for (int rb = 0; rb < RX_RB; ++rb) {
      xb[rb] = slab_frag(0, rb);
      xs[rb] = slab_scale(0, rb);
    }
    ScB sbs;
    load_sb(cur, sbs);

    // ---- one slab step of GEMM1 pass PH (0: A, 1: B): slab t = 6 m + K of
    // the pass (t + NSP in the tile's slab stream for pass B), K % 3 its
    // buffer. Slab t+1 is quantised into its buffer and slab t+3's loads go
    // out, then the slab's k-step; the barrier after it makes slab t+1
    // visible for the next step's operands, which are read row block by row
    // block, and means every wave is done with slab t-1, whose buffer the
    // next step fills.
    auto slab_step = [&](auto ph_tag, auto k_tag, int m, auto& sg, auto& su, const auto& sc)
        __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value, K = decltype(k_tag)::value;
      constexpr int F = PH == 0 ? FA : FB;
      constexpr int sbn = (K + 1) % 3;
      const int t = (PH == 0 ? 0 : NSP) + 6 * m + K;
      slab_store(sbn, sv[(K + 1) & 1]);
      slab_load(t + 3, sv[(K + 1) & 1]);
      const int kb = 6 * m + K;   // k-step of the pass (compile-time once unrolled)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb)
#pragma unroll
        for (int i = 0; i < F; ++i) {
          // the pass's first k-step takes a zero accumulator operand
          f32x16& acc = (i & 1) ? su[rb][i >> 1] : sg[rb][i >> 1];
          acc = rx_mfma_s(kb & 3, ring[(kb * F + i) % RX_RING], xb[rb], sc.w[i >> 1][i & 1][kb >> 2], xs[rb],
                          kb == 0 ? f32x16{} : acc);
        }
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int pos = kb * F + i;
        refill(ring[pos % RX_RING], std::integral_constant<int, PH>{}, pos % RX_RING, pos / RX_RING + 1);
      }
      // the k-step's products are taken here: the compiler would otherwise
      // sink the MFMAs (pure operations) down to the accumulators' use after
      // the pass, keeping every k-step's operands live until then
#pragma unroll
      for (int rb = 0; rb < RX_RB; ++rb)
#pragma unroll
        for (int h = 0; h < F / 2; ++h) asm volatile("" : "+a"(sg[rb][h]), "+a"(su[rb][h]));
      __syncthreads();
      if (t + 1 < NSL) {
#pragma unroll
        for (int rb = 0; rb < RX_RB; ++rb) {
          xb[rb] = slab_frag(sbn, rb);
          xs[rb] = slab_scale(sbn, rb);
        }
      }
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
          if (((ot >> 5) & 1) == 0) usc[row * USC + nb] = (uint8_t)(k + 127);
          // one accumulator block at a time: the scheduler would otherwise
          // move every accumulator to VGPRs at once
          __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ================= GEMM1 pass A =================
    {
      f32x16 sg[RX_RB][HA], su[RX_RB][HA];
#pragma unroll
      for (int m = 0; m < NSP / 6; ++m) {
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, m, sg, su, sa);
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, m, sg, su, sa);
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, m, sg, su, sa);
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{}, m, sg, su, sa);
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{}, m, sg, su, sa);
        slab_step(std::integral_constant<int, 0>{}, std::integral_constant<int, 5>{}, m, sg, su, sa);
      }
      store_u(HA * wave, sg, su, std::integral_constant<int, HA>{});
    }
    ScC scc;
    load_sc(cur, 0, scc);
    // ================= GEMM1 pass B =================
    fresh();
    {
      f32x16 sg[RX_RB][HBB], su[RX_RB][HBB];
#pragma unroll
      for (int m = 0; m < NSP / 6; ++m) {
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, m, sg, su, sbs);
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, m, sg, su, sbs);
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}, m, sg, su, sbs);
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{}, m, sg, su, sbs);
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{}, m, sg, su, sbs);
        slab_step(std::integral_constant<int, 1>{}, std::integral_constant<int, 5>{}, m, sg, su, sbs);
      }
      store_u(4 * HA + HBB * wave, sg, su, std::integral_constant<int, HBB>{});
    }
    __syncthreads();   // U complete

    // the claim of the tile after next goes out now (read after the epilogue)
    int qnext = 0;
    if (tid == 0) qnext = atomicAdd(&a.qhead[qx], 1);

    // ================= GEMM2 parts, each with its epilogue =================
    auto gemm2_part = [&](auto ph_tag, f32x16 (&o)[RX_RB][FC], const ScC& s) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value;
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
    // gate * O of row block rb -> staging rows (stride HS)
    auto stage_rb = [&](int rb, f32x16 (&o)[RX_RB][FC]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < FC; ++j) asm volatile("" : "+a"(o[rb][j]));
      const float g = rowg[buf][rb * 32 + (ot & 31)];
#pragma unroll
      for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 w2;
          w2.x = pack_bf16x2(g * o[rb][j][4 * g4], g * o[rb][j][4 * g4 + 1]);
          w2.y = pack_bf16x2(g * o[rb][j][4 * g4 + 2], g * o[rb][j][4 * g4 + 3]);
          *reinterpret_cast<uint2*>(&stg[(ot & 31) * HS + (2 * wave + j) * 32 + 8 * g4 + 4 * ((ot >> 5) & 1)]) = w2;
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
        v[k] = *reinterpret_cast<const v4u*>(&stg[r * HS + c8 * 8]);
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
      for (int rb = 0; rb < RX_RB; ++rb) {
        stage_rb(rb, o);
        __syncthreads();
        store_rows(rb * 32, PH - 2);
        __syncthreads();
      }
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
  if (a.hidden != 384 || a.wrec < mx_rec_dwords(768, 384)) return hipErrorInvalidValue;
  workers &= ~7;
  const int grid = (workers <= 0 || tiles <= workers) ? tiles : workers;
  hipLaunchKernelGGL((routed_mx_kernel<768, 384>), dim3(grid), dim3(RX_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tmx
