// tmx_routed.hip -- the grouped routed-expert MLP of the Sparse-Pertoken MoE
// (TokenMixer-Large summary Eq. 19, section 2.5.1 MoEGroupedSwiGLU) for wide
// rows (W = 768, h_e = 384; W = 512, h_e = 256), on gfx950 bf16 MFMA.
//
// Why a kernel of its own: in the general fused MLP kernel a W = 768 tile has
// 64 rows (its GEMM2 accumulators, 64 x 768 fp32, fill the AGPRs), so every
// weight fragment fed from L2 serves two 32-row MFMA blocks, and that weight
// stream, not the MFMA rate, bounds the routed launch (at W = 512 the 4-wave
// fused tile also holds 64 rows). Here a tile has BM = 128 rows of one
// (position, expert) bucket, and each weight fragment serves four MFMA
// blocks, which halves the weight bytes per FLOP. The accumulators of 128
// rows do not fit at once either, so a tile runs in phases that each stay
// within the 256 AGPRs (shown for W = 768, h_e = 384):
//
//   GEMM1 A  S_gate, S_up for hidden blocks [8 blocks of 32] (2 per wave,
//            256 accumulator registers), K-outer: the rows' x_hat columns
//            stream through LDS in 64-column slabs;
//   U(A)     rho(silu(S_gate) * S_up) -> LDS U [128, h_e];
//   GEMM1 B  the other 4 hidden blocks (1 per wave), x_hat streamed again;
//   U(B)     -> LDS U;
//   GEMM2 0  O [128, 0:384) = U @ W_down[:, 0:384) (3 column blocks per wave);
//   out 0    gate * O -> bf16, staged 32 rows at a time through two free slab
//            buffers and written as whole 16-byte units of the rows' slots of
//            the expert-output buffer;
//   GEMM2 1  O [128, 384:768) ... out 1 (staged through the U region).
//
// At h_e = 256 pass A covers the whole hidden (no pass B: x_hat is read once)
// and each GEMM2 half has 2 column blocks per wave.
//
// The second x_hat pass costs 196 KB of L2/last-level-cache reads per tile
// against the 1.7 MB of expert weights every tile streams.
//
// Pipelines. Weight fragments stream through a register ring (24 slots at
// W = 768, 16 at W = 512) in one order per tile (GEMM1 A, GEMM1 B, GEMM2 0,
// GEMM2 1) that runs on into the next tile; a slot is refilled as soon as its
// four MFMAs have issued. x_hat slabs (24 per tile at W = 768: 12 per GEMM1
// pass; 8 at W = 512) run through three LDS buffers (four at W = 512, so
// that a tile's slab count is a whole number of buffer turns): at slab step
// s, slab s+1 goes from registers to LDS and slab s+3's loads go out (two
// register sets, so a load has two slab steps to land); the last three slab
// steps of a tile load the next tile's first slabs, which wait in LDS buffer
// 0 and registers through GEMM2.
#include <type_traits>

#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int RT_NT = 256;   // 4 waves
constexpr int RT_RB = 4;     // 32-row blocks per tile
constexpr int RT_BM = 32 * RT_RB;
constexpr int RT_SC = 64;    // columns per x_hat slab
constexpr int RT_RSRC_W3 = 0x00020000;   // buffer resource word 3: raw 32-bit data, no swizzle
// cache policy of the second pass's x_hat loads (the rows' last use) and of
// the gated-output stores: streaming (non-temporal), which keeps the expert
// weights, re-read by every tile of a bucket, in L2
constexpr int RT_NT_POLICY = 2;

// 16 bytes as a native vector: arrays of it stay in registers (arrays of the
// struct type uint4 are copied with memcpy, which can leave them in scratch)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u rt_ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }

__device__ __forceinline__ f32x16 rt_mfma(const v4u& a, const v4u& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// z * sigmoid(z) with the hardware exp and reciprocal; rounded to bf16 next
__device__ __forceinline__ float rt_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <int W, int HE>
struct RtShape {
  static constexpr int BM = RT_BM;
  static constexpr int HA = 2;                    // hidden blocks per wave, GEMM1 pass A
  static constexpr int HBB = HE / 128 - HA;       // ... pass B (none at h_e = 256)
  static constexpr int NOH = W / 256;             // output blocks per wave and GEMM2 half
  static constexpr int NSP = W / RT_SC;           // slabs per GEMM1 pass
  static constexpr int NSL = (HBB > 0 ? 2 : 1) * NSP;   // slab steps per tile
  // x_hat slab buffers in LDS and the slab-step group: slab t sits in buffer
  // t % NBUF and register set t % 2, and a tile's NSL slab steps must be
  // whole groups so that the next tile's slab 0 lands in buffer 0, set 0
  static constexpr int NBUF = NSL % 3 == 0 ? 3 : 4;
  static constexpr int G = NBUF == 3 ? 6 : 4;
  static constexpr int RING = W == 768 ? 24 : 16; // weight fragments in flight per wave
  static constexpr int KB1 = W / 16;              // GEMM1 k-steps per pass
  static constexpr int KB2 = HE / 16;             // GEMM2 k-steps per half
  static constexpr int FA = 2 * HA, FB = 2 * HBB, FC = NOH;   // fragments per k-step
  static constexpr int LA = KB1 * FA, LB = KB1 * FB, LC = KB2 * FC;   // fragments per phase
  static constexpr int US = HE + 8;               // U row stride (bf16): rows 16 B apart in banks
  static constexpr int HS = W / 2 + 8;            // staged half-row stride (bf16)
  static constexpr int SLAB = BM * RT_SC;         // bf16 per slab buffer
  static constexpr int SU = BM * RT_SC / 8 / RT_NT;   // slab units per lane
  static_assert(HE % 128 == 0 && HBB >= 0 && HBB <= 2, "one or two GEMM1 passes of at most 2 hidden blocks per wave");
  static_assert(W % 256 == 0 && W % RT_SC == 0 && NSP % G == 0 && NSL % NBUF == 0,
                "slab steps run in whole groups, and pass B starts at a group");
  static_assert((BM * RT_SC / 8) % RT_NT == 0, "slab units per lane");
  static_assert(LA % RING == 0 && LB % RING == 0 && LC % RING == 0 && RING % FA == 0 &&
                (FB == 0 || RING % FB == 0) && RING % FC == 0,
                "every phase is whole turns of the ring, each of whole k-steps");
  static_assert(KB2 % 4 == 0, "GEMM2 k-steps run in groups of four");
  static_assert(32 * HS * 2 <= 2 * SLAB * 2, "a staged 32-row half fits in two slab buffers");
  static_assert(BM * HS <= BM * US, "a staged 128-row half fits in the U region");
  static_assert(NBUF * SLAB * 2 + BM * US * 2 + 3 * 2 * BM * 4 + 16 <= 160 * 1024, "LDS budget");
};

template <int W, int HE>
__global__ __launch_bounds__(RT_NT, 1) void routed_kernel(const MlpArgs a) {
  using S = RtShape<W, HE>;
  constexpr int BM = S::BM, HA = S::HA, HBB = S::HBB, NOH = S::NOH, NSP = S::NSP, NSL = S::NSL;
  constexpr int NBUF = S::NBUF, G = S::G, RING = S::RING;
  constexpr int KB1 = S::KB1, KB2 = S::KB2, FA = S::FA, FB = S::FB, FC = S::FC;
  constexpr int LA = S::LA, LB = S::LB, LC = S::LC, US = S::US, HS = S::HS, SLAB = S::SLAB, SU = S::SU;

  __shared__ __attribute__((aligned(16))) uint16_t slabs[NBUF * SLAB];
  __shared__ __attribute__((aligned(16))) uint16_t us[BM * US];
  __shared__ int rowb[2][BM];      // sample row of each tile row (-1: padding)
  __shared__ int rowgi[2][BM];     // expert-output row (b, p, slot)
  __shared__ float rowg[2][BM];    // gate of each tile row
  __shared__ int claim;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Lane-dependent address arithmetic reads `ot`, an opaque copy of the
  // thread index that is made anew before each phase: the compiler cannot
  // then hoist one phase's addresses out of the tile loop (they would stay
  // live, in registers or spilled, through every other phase).
  int ot = tid;
  auto fresh = [&]() __attribute__((always_inline)) { asm volatile("" : "+v"(ot)); };

  // ---- tile queues (one per XCD over its positions when P % 8 == 0): entry
  // k is the k-th non-empty tile of the queue's positions in order; the
  // bucket kernel zeroes the heads
  const bool split_q = (a.P & 7) == 0;
  const int qx = split_q ? (int)(blockIdx.x & 7) : 0;
  const int NPX = split_q ? (a.P >> 3) : a.P;
  struct Tile {
    int p, group, start, nrows;
  };
  // the decoded values are the same in every lane; readfirstlane keeps the
  // weight addresses in scalar registers
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
    for (int r = tid; r < BM; r += RT_NT) {
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
  //   1  GEMM1 B: hidden block 4 HA + HBB wave + h
  //   2  GEMM2 0: k-step kb, output block NOH wave + j
  //   3  GEMM2 1: output block W / 64 + NOH wave + j
  //   4  the next tile's phase 0
  // A super-step is one turn of the ring (12 fragments: 3 k-steps of phase
  // 0, 6 of phase 1, 4 of a GEMM2 half). Slot i holds fragment i of the
  // current super-step and is refilled with fragment i of the next one,
  // which may belong to the next phase: both addresses are formed and one is
  // selected, so every refill is one unconditional load (a load on one path
  // only makes the compiler wait for every load in flight where the paths
  // join). i is a compile-time constant; only the super-step index is not.
  // The weights of a bucket, and x_hat, are read through buffer resources:
  // the lane's part of an address is a 32-bit VGPR offset (lane and wave),
  // the fragment's a constant byte offset, so no load needs 64-bit address
  // arithmetic (which, once unrolled, the compiler would keep in scalar
  // registers for hundreds of fragments).
  constexpr uint32_t GU_BYTES = (HE / 32) * KB1 * 2 * FRAG_ELEMS * 2;   // gate|up fragments of a bucket
  constexpr uint32_t WD_BYTES = KB2 * (W / 32) * FRAG_ELEMS * 2;        // down fragments of a bucket
  auto rsrc = [](const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RT_RSRC_W3);
  };
  __amdgpu_buffer_rsrc_t cgu, cwd, ngu, nwd;
  auto bases = [&](const Tile& T, __amdgpu_buffer_rsrc_t& gu, __amdgpu_buffer_rsrc_t& wd) {
    gu = rsrc(a.wgu + (size_t)T.group * (GU_BYTES / 2), GU_BYTES);
    wd = rsrc(a.wd + (size_t)T.group * (WD_BYTES / 2), WD_BYTES);
  };
  // per-lane byte offsets of the phases (lane and wave parts)
  auto voff_gu = [&](int nb0) -> uint32_t { return (uint32_t)(ot & 63) * 16u + (uint32_t)nb0 * KB1 * 2048u; };
  auto voff_wd = [&]() -> uint32_t { return (uint32_t)(ot & 63) * 16u + (uint32_t)(NOH * wave) * 1024u; };
  // fragment at position pos of phase ph (ph and pos compile-time once unrolled)
  auto wload = [&](int ph, int pos) __attribute__((always_inline)) -> v4u {
    if (ph == 0 || ph == 4) {
      const int kb = pos / FA, ii = pos % FA;
      const int c = (((ii >> 1) * KB1 + kb) * 2 + (ii & 1)) * 1024;
      return __builtin_amdgcn_raw_buffer_load_b128(ph == 0 ? cgu : ngu, voff_gu(HA * wave), c, 0);
    }
    if (HBB > 0 && ph == 1) {
      constexpr int FBn = FB > 0 ? FB : 1;
      const int kb = pos / FBn, ii = pos % FBn;
      const int c = (((ii >> 1) * KB1 + kb) * 2 + (ii & 1)) * 1024;
      return __builtin_amdgcn_raw_buffer_load_b128(cgu, voff_gu(4 * HA + HBB * wave), c, 0);
    }
    const int kb = pos / FC, j = pos % FC;
    const int c = (kb * (W / 32) + (ph == 3 ? W / 64 : 0) + j) * 1024;
    return __builtin_amdgcn_raw_buffer_load_b128(cwd, voff_wd(), c, 0);
  };
  constexpr int SA = LA / RING, SB = LB / RING, SC = LC / RING;   // super-steps per phase
  // slot i of phase PH, refilled for super-step sn (past the phase: the next
  // one, which after pass A is GEMM2 when there is no pass B)
  auto refill = [&](v4u& dst, auto ph_tag, int i, int sn) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_tag)::value;
    constexpr int NSS = PH == 0 ? SA : PH == 1 ? SB : SC;
    constexpr int NPH = (PH == 0 && HBB == 0) ? 2 : PH + 1;
    dst = sn < NSS ? wload(PH, sn * RING + i) : wload(NPH, (sn - NSS) * RING + i);
  };
  v4u ring[RING];

  // ---- x_hat slabs: unit u = tid + 256 i of a slab is row u / 8, 16-byte
  // chunk u % 8 of the slab's 64 columns, stored at chunk (u % 8) ^ (row % 8)
  // of its LDS row (XOR swizzle: the fragment reads of 8 consecutive rows hit
  // 8 different bank groups). x_hat stays below 4 GiB (the host checks its
  // size), so a lane keeps one 32-bit byte offset per row of its units, for
  // this tile and the next.
  uint32_t roff[SU], roffn[SU];
  auto slab_rows = [&](int p, int buf, uint32_t* ro) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RT_NT;
      const int b = rowb[buf][u >> 3];
      ro[i] = (((uint32_t)p * (uint32_t)a.B + (uint32_t)(b < 0 ? 0 : b)) * (uint32_t)W + (uint32_t)(u & 7) * 8u) * 2u;
    }
  };
  // slab t of the slab stream (t >= NSL: the next tile's slab t - NSL)
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.xhat, (uint32_t)((uint64_t)a.P * a.B * W * 2));
  auto slab_load = [&](int t, v4u* v) __attribute__((always_inline)) {
    const bool nxt = t >= NSL;
    const int col = (nxt ? t - NSL : (t >= NSP ? t - NSP : t)) * RT_SC * 2;
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const uint32_t o = nxt ? roffn[i] : roff[i];
      v[i] = (t >= NSP && !nxt) ? __builtin_amdgcn_raw_buffer_load_b128(xr, o, col, RT_NT_POLICY)
                                : __builtin_amdgcn_raw_buffer_load_b128(xr, o, col, 0);
    }
  };
  auto slab_store = [&](int sb, const v4u* v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = ot + i * RT_NT, r = u >> 3;
      *reinterpret_cast<v4u*>(&slabs[sb * SLAB + r * RT_SC + (((u & 7) ^ (r & 7)) * 8)]) = v[i];
    }
  };
  // B operand of row block rb, k-step q of a slab: row 32 rb + l32, columns
  // 16 q + 8 h32 .. + 8
  auto slab_frag = [&](int sb, int rb, int q) -> v4u {
    const int r = rb * 32 + (ot & 31);
    return *reinterpret_cast<const v4u*>(&slabs[sb * SLAB + r * RT_SC + (((2 * q + ((ot >> 5) & 1)) ^ (r & 7)) * 8)]);
  };
  // B operand of GEMM2 k-step kb: U row 32 rb + l32, hidden 16 kb + 8 h32 .. + 8
  auto u_frag = [&](int rb, int kb) -> v4u {
    return *reinterpret_cast<const v4u*>(&us[(rb * 32 + (ot & 31)) * US + kb * 16 + ((ot >> 5) & 1) * 8]);
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
  {
    v4u s0[SU];
    slab_load(0, s0);
    slab_load(1, sv[1]);
    slab_load(2, sv[0]);
#pragma unroll
    for (int f = 0; f < RING; ++f) ring[f] = wload(0, f);
    slab_store(0, s0);
  }
  __syncthreads();

  while (true) {
    fresh();
    v4u xb[RT_RB];
#pragma unroll
    for (int rb = 0; rb < RT_RB; ++rb) xb[rb] = slab_frag(0, rb, 0);

    // ---- one slab step of GEMM1 pass PH (0: A, 1: B): slab t = 6 m + K of
    // the pass (m runtime, K compile-time; t + NSP in the tile's slab stream
    // for pass B). K % NBUF is the slab's buffer. Slab t+1 goes from registers
    // to its buffer and slab t+3's loads go out, then the slab's 4 k-steps.
    // The barrier before the last k-step makes slab t+1 visible (that step
    // prefetches its first fragments) and means every wave is done with slab
    // t-1, whose buffer the next step fills.
    auto slab_step = [&](auto ph_tag, auto k_tag, int m, auto& sg, auto& su) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value, K = decltype(k_tag)::value;
      constexpr int F = PH == 0 ? FA : FB;
      constexpr int sb = K % NBUF, sbn = (K + 1) % NBUF;
      const int t = (PH == 0 ? 0 : NSP) + G * m + K;             // slab of the tile's stream
      slab_store(sbn, sv[(K + 1) & 1]);
      slab_load(t + 3, sv[(K + 1) & 1]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q == 3) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 24 m + 4 K + q of the pass (all compile-time once unrolled).
        // Row block by row block: once a block's F MFMAs have issued, its
        // x_hat fragment is replaced by the next k-step's (the next slab's on
        // the last step), so one register set serves both; the weight
        // fragments' slots are refilled after the last block.
        const int kb = 4 * (G * m + K) + q;
#pragma unroll
        for (int rb = 0; rb < RT_RB; ++rb) {
#pragma unroll
          for (int i = 0; i < F; ++i) {
            // the pass's first k-step takes a zero accumulator operand: no
            // separate clearing, which the compiler would hoist into the
            // previous phase (evicting its live accumulators to VGPRs)
            f32x16& acc = (i & 1) ? su[rb][i >> 1] : sg[rb][i >> 1];
            acc = rt_mfma(ring[(kb * F + i) % RING], xb[rb], kb == 0 ? f32x16{} : acc);
          }
          if (q < 3) xb[rb] = slab_frag(sb, rb, q + 1);
          else if (t + 1 < NSL) xb[rb] = slab_frag(sbn, rb, 0);
        }
#pragma unroll
        for (int i = 0; i < F; ++i) {
          const int pos = kb * F + i;
          refill(ring[pos % RING], std::integral_constant<int, PH>{}, pos % RING, pos / RING + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // U of a pass's hidden blocks (block nb0 + h of the wave) -> LDS
    auto store_u = [&](int nb0, auto& sg, auto& su, auto nh_tag) __attribute__((always_inline)) {
      constexpr int NH = decltype(nh_tag)::value;
#pragma unroll
      for (int rb = 0; rb < RT_RB; ++rb)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float uv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) uv[e] = rt_silu(sg[rb][h][4 * g4 + e]) * su[rb][h][4 * g4 + e];
            uint2 w2;
            w2.x = pack_bf16x2(uv[0], uv[1]);
            w2.y = pack_bf16x2(uv[2], uv[3]);
            *reinterpret_cast<uint2*>(&us[(rb * 32 + (ot & 31)) * US + (nb0 + h) * 32 + 8 * g4 + 4 * ((ot >> 5) & 1)]) = w2;
            // one accumulator quarter at a time: the scheduler would otherwise
            // move every accumulator to VGPRs at once
            __builtin_amdgcn_sched_barrier(0);
          }
    };

    // one group of G slab steps of pass PH (K = 0 .. G-1, compile-time)
    auto slab_group = [&](auto ph_tag, int m, auto& sg, auto& su) __attribute__((always_inline)) {
      slab_step(ph_tag, std::integral_constant<int, 0>{}, m, sg, su);
      slab_step(ph_tag, std::integral_constant<int, 1>{}, m, sg, su);
      slab_step(ph_tag, std::integral_constant<int, 2>{}, m, sg, su);
      slab_step(ph_tag, std::integral_constant<int, 3>{}, m, sg, su);
      if constexpr (G == 6) {
        slab_step(ph_tag, std::integral_constant<int, 4>{}, m, sg, su);
        slab_step(ph_tag, std::integral_constant<int, 5>{}, m, sg, su);
      }
    };
    // ================= GEMM1 pass A =================
    {
      f32x16 sg[RT_RB][HA], su[RT_RB][HA];
#pragma unroll
      for (int m = 0; m < NSP / G; ++m) slab_group(std::integral_constant<int, 0>{}, m, sg, su);
      store_u(HA * wave, sg, su, std::integral_constant<int, HA>{});
    }
    // ================= GEMM1 pass B (h_e > 256) =================
    fresh();
    if constexpr (HBB > 0) {
      f32x16 sg[RT_RB][HBB], su[RT_RB][HBB];
#pragma unroll
      for (int m = 0; m < NSP / G; ++m) slab_group(std::integral_constant<int, 1>{}, m, sg, su);
      store_u(4 * HA + HBB * wave, sg, su, std::integral_constant<int, HBB>{});
    }
    __syncthreads();   // U complete

    // the claim of the tile after next goes out now (read after the epilogue)
    int qnext = 0;
    if (tid == 0) qnext = atomicAdd(&a.qhead[qx], 1);

    // ================= GEMM2, two column halves, each with its epilogue =================
    v4u ub[RT_RB];
    auto gemm2_half = [&](auto ph_tag, f32x16 (&o)[RT_RB][NOH]) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value;
#pragma unroll
      for (int rb = 0; rb < RT_RB; ++rb) ub[rb] = u_frag(rb, 0);
#pragma unroll
      for (int kb = 0; kb < KB2; ++kb) {
        __builtin_amdgcn_sched_barrier(0);
        // past the last k-step the prefetch reads k-step 0 again (unused)
        const int kn = kb + 1 < KB2 ? kb + 1 : 0;
#pragma unroll
        for (int rb = 0; rb < RT_RB; ++rb) {
#pragma unroll
          for (int j = 0; j < FC; ++j)
            o[rb][j] = rt_mfma(ring[(kb * FC + j) % RING], ub[rb], kb == 0 ? f32x16{} : o[rb][j]);
          ub[rb] = u_frag(rb, kn);
        }
#pragma unroll
        for (int j = 0; j < FC; ++j) {
          const int pos = kb * FC + j;
          refill(ring[pos % RING], std::integral_constant<int, PH>{}, pos % RING, pos / RING + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // gate * O of row block rb, half c -> staging rows [32 r0 ...) (stride HS)
    auto stage_rb = [&](uint16_t* stg, int rs, int rb, f32x16 (&o)[RT_RB][NOH]) __attribute__((always_inline)) {
      // the block's accumulators stay in AGPRs up to here (the compiler
      // otherwise copies every block's to VGPRs at once, the kernel's
      // register peak)
#pragma unroll
      for (int j = 0; j < NOH; ++j) asm volatile("" : "+a"(o[rb][j]));
      const float g = rowg[buf][rb * 32 + (ot & 31)];
#pragma unroll
      for (int j = 0; j < NOH; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 w2;
          w2.x = pack_bf16x2(g * o[rb][j][4 * g4], g * o[rb][j][4 * g4 + 1]);
          w2.y = pack_bf16x2(g * o[rb][j][4 * g4 + 2], g * o[rb][j][4 * g4 + 3]);
          *reinterpret_cast<uint2*>(&stg[(rs + (ot & 31)) * HS + (NOH * wave + j) * 32 + 8 * g4 + 4 * ((ot >> 5) & 1)]) = w2;
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    // staged rows [row0, row0 + nr) of half c -> the expert-output rows
    constexpr int U8H = W / 16;   // 16-byte units per half row
    // (unrolled, in batches: every batch's LDS reads go out before its
    // stores, so a lane waits once per batch, not once per unit)
    auto store_rows = [&](const uint16_t* stg, int row0, auto nr_tag, int c) __attribute__((always_inline)) {
      constexpr int NR = decltype(nr_tag)::value, NU = NR * U8H / RT_NT;
      constexpr int BATCH = NU % 8 == 0 ? 8 : NU;
      static_assert((NR * U8H) % RT_NT == 0 && NU % BATCH == 0, "output units per lane");
#pragma unroll
      for (int i0 = 0; i0 < NU; i0 += BATCH) {
        v4u v[BATCH];
        int gi[BATCH], c8s[BATCH];
        bool ok[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int u = ot + (i0 + k) * RT_NT, r = u / U8H, c8 = u - r * U8H, row = row0 + r;
          v[k] = *reinterpret_cast<const v4u*>(&stg[r * HS + c8 * 8]);
          ok[k] = rowb[buf][row] >= 0;
          gi[k] = rowgi[buf][row];
          c8s[k] = c8;
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k)
          if (ok[k])
            __builtin_nontemporal_store(v[k], reinterpret_cast<v4u*>(a.part + (size_t)gi[k] * W + c * (W / 2) + c8s[k] * 8));
      }
    };
    {
      fresh();
      f32x16 o[RT_RB][NOH];
      gemm2_half(std::integral_constant<int, 2>{}, o);
      fresh();
      // half 0 goes out through slab buffers 1 and 2 (free until the next
      // tile), 32 rows at a time, while U is still needed
      uint16_t* stg = slabs + SLAB;
#pragma unroll
      for (int rb = 0; rb < RT_RB; ++rb) {
        stage_rb(stg, 0, rb, o);
        __syncthreads();
        store_rows(stg, rb * 32, std::integral_constant<int, 32>{}, 0);
        __syncthreads();
      }
    }
    {
      fresh();
      f32x16 o[RT_RB][NOH];
      gemm2_half(std::integral_constant<int, 3>{}, o);
      fresh();
      __syncthreads();   // every wave's U reads done: U becomes the stage
#pragma unroll
      for (int rb = 0; rb < RT_RB; ++rb) stage_rb(us, rb * 32, rb, o);
      if (tid == 0) claim = qnext;
      __syncthreads();
      store_rows(us, 0, std::integral_constant<int, BM>{}, 1);
      __syncthreads();
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

template <int W, int HE>
hipError_t launch_rt(const MlpArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((routed_kernel<W, HE>), dim3(grid), dim3(RT_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int routed_wide_rows(int W, int h_e) { return ((W == 768 && h_e == 384) || (W == 512 && h_e == 256)) ? RT_BM : 0; }

hipError_t launch_routed_wide(const MlpArgs& a, int tiles, int workers, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  workers &= ~7;
  const int grid = (workers <= 0 || tiles <= workers) ? tiles : workers;
  // (routed_wide_rows admits one width per expert hidden size)
  if (a.hidden == 384) return launch_rt<768, 384>(a, grid, s);
  if (a.hidden == 256) return launch_rt<512, 256>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace tmx
