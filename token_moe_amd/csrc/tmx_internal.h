// tmx_internal.h -- argument blocks and launchers shared between the host
// library (tmx_host.hip) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tmx_device.h"

namespace tmx {

enum MlpMode { MLP_DENSE = 0, MLP_ROUTED = 1, MLP_SHARED = 2 };

// hidden units per chunk of the fused MLP (hidden sizes must be multiples)
constexpr int MLP_HC = 128;

// B-operand fragment shapes of the packer
enum FragShape { FRAG_16x16x32 = 0, FRAG_32x32x16 = 1 };

// One launch of the fused per-position SwiGLU MLP over row tiles:
//   DENSE : out = rho(resid + SwiGLU_p(rho(RMSNorm(x_p))) [+ extra])
//   ROUTED: part[b,p,s] = rho(gate[b,p,s] * SwiGLU_{p,e}(xhat[p, b]))   (bucket rows)
//   SHARED: out = rho(resid + SwiGLU_p,sh(xhat[p,b]) + sum_s part[b,p,s] [+ extra])
struct MlpArgs {
  int B;               // batch rows
  int P;               // positions of the sub-layer
  int hidden;          // hidden size of the MLP (dense h, h_e or h_s)
  RowMap map;          // block-layout map of x / resid / extra / out
  float eps;
  const uint16_t* x;       // DENSE source, [B, T, D]
  const float* gain;       // DENSE: RMSNorm gain [W]
  const uint16_t* xhat;    // ROUTED / SHARED source, [P][B][W]
  const uint8_t* xq8;      // the MXFP8 wide routed kernel's source: x_hat in MXFP8
  const uint8_t* xe8;      // (RouteArgs::xq8, xe8)
  const uint16_t* wgu;     // packed gate|up fragments
  const uint16_t* wd;      // packed down fragments
  const uint16_t* resid;   // DENSE / SHARED
  const uint16_t* extra;   // nullable
  uint16_t* out;           // DENSE / SHARED
  int top_k, E, max_tiles;
  const int* rows;         // ROUTED: [P][B*top_k] bucket entries (b*top_k + slot)
  const int4* tiles;       // ROUTED: [P][max_tiles] (expert, start, count, 0)
  const int* ntiles;       // ROUTED: [P]
  const float* gate;       // ROUTED: [B][P][top_k]
  uint16_t* part;          // ROUTED writes / SHARED reads, [B][P][top_k][W] bf16
                           // (gated expert outputs, each rounded to bf16)
  int* qhead;              // ROUTED: [8] per-XCD tile-queue heads, zero at launch
  int rtiles;              // DENSE / SHARED: row tiles per position unit
  int pair;                // DENSE / SHARED: 1 = a tile holds BM/2 rows of each of two
                           // adjacent positions (2q in rows [0, BM/2), 2q+1 above)
  const uint32_t* wsc;     // MXFP8: weight scale records (see launch_pack_mx)
  int wrec;                // MXFP8: dwords per lane record (mx_rec_dwords)
  int ileave;              // DENSE / SHARED, unpaired: positions 2q and 2q+1 alternate
                           // in the tile order (row tile t of 2q, of 2q+1, t+1 of 2q, ...)
  int stagger;             // clocks that the late half of the workgroups waits before
                           // its first tile (0 = none): every other workgroup of an
                           // XCD, or with two workgroups per CU the second of each CU
};

struct RouteArgs {
  int B, P, E, top_k;
  float alpha, eps;
  RowMap map;
  const uint16_t* x;       // block layout [B, T, D]
  const float* gain;       // [W]
  const uint16_t* wr;      // packed router fragments
  uint16_t* xhat;          // [P][B][W] (nullable)
  uint8_t* xq8;            // nullable: x_hat in MXFP8, E4M3 codes [P][B][W] ...
  uint8_t* xe8;            // ... and exponents [P][B][W/32] (bias 127), one per 32 columns
  int32_t* idx;            // [B][P][top_k]
  float* gate;             // [B][P][top_k]
  int* hist;               // nullable: [P][ceil(B/64)][E] choices per 64-row chunk
};

struct BucketArgs {
  int B, P, E, top_k, bm, max_tiles;
  const int32_t* idx;      // [B][P][top_k]
  int* rows;               // [P][B*top_k]
  int4* tiles;             // [P][max_tiles]
  int* ntiles;             // [P]
  int* counts;             // [P][E]
  const int* hist;         // [P][ceil(B/64)][E] from norm_route
  int* qhead;              // [8] tile-queue heads of the routed MLP, zeroed here
};

// bf16 launchers (return hipError_t of the launch)
// rows per tile of the MLP kernel for a mode (MlpMode) and width
int mlp_bm(int mode, int W);
bool mlp_width_supported(int W);
// tiles = P * (rtiles or max_tiles); the grid is min(tiles, (workers & ~7) *
// workgroups per CU): each workgroup walks tiles blockIdx.x, blockIdx.x +
// grid, ...
hipError_t launch_mlp(int mode, int W, const MlpArgs& a, int tiles, int workers, hipStream_t s);
// routed experts at W = 768, h_e = 384 (tmx_routed.hip): rows per bucket tile
// (0 where that kernel does not apply) and its launch (grid as launch_mlp,
// ROUTED arguments)
int routed_wide_rows(int W, int h_e);
hipError_t launch_routed_wide(const MlpArgs& a, int tiles, int workers, hipStream_t s);
// its MXFP8 form (tmx_routed_mx.hip): same tiles and arguments, weights and
// scale records from launch_pack_mx
int routed_wide_mx_rows(int W, int h_e);
hipError_t launch_routed_wide_mx(const MlpArgs& a, int tiles, int workers, hipStream_t s);
// whether DENSE / SHARED tiles of this mode and width may hold two adjacent positions
bool mlp_pairs_positions(int mode, int W);
// workgroups of the MLP kernel resident per CU for a mode and width
int mlp_workgroups_per_cu(int mode, int W);
hipError_t launch_norm_route(int W, const RouteArgs& a, hipStream_t s);
hipError_t launch_bucket(const BucketArgs& a, hipStream_t s);
// Repack G row-major [K, N] bf16 matrices into MFMA B-operand fragments of
// shape `frag` (FragShape). layout 0: gate|up interleave (`which` = 0 gate,
// 1 up), frag = ((g*NB + nb)*KB + kb)*2 + which; layout 1: k-major,
// frag = (g*KB + kb)*NB + nb; layout 2: n-major, frag = (g*NB + nb)*KB + kb.
hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int G, int K, int N, int layout,
                       int which, int frag, hipStream_t s);
// MXFP8 weights of the MXFP8 MLP kernels (sub-layer width W in {256, 512, 768}):
// G row-major [K, N] bf16 matrices -> E4M3 codes in 32 x 64 fragments of the
// v_mfma_scale_f32_32x32x64_f8f6f4 A operand (two 1 KiB halves: lane l holds
// row l % 32, bytes 0-15 of K-block 0 and 16-31 of K-block 1 of the 64-K step,
// k = 16 * (l / 32) + j within the block) plus E8M0 scales (one per column and
// 32-element K-block) in per-lane records `rec` [G][4 waves][64 lanes][R]
// dwords, R = mx_rec_dwords(W, hidden). With DW = W / 256, hidden chunk c
// (128 units) owns dwords [3 DW c, 3 DW (c + 1)): gate (m = 0), up (m = 1)
// and down (m = 2) take DW dwords each, byte q of matrix m at dword
// 3 DW c + DW m + q / 4, byte q % 4. Gate/up: q = K-step s of the 64-K steps
// along W, the scale of K-block 2s + l / 32 of column 32 (4c + wave) + l % 32.
// Down: q = 2j + t, the scale of column 32 (NBO wave + j) + l % 32 (NBO = W /
// 128 column blocks per wave) and hidden block 4c + 2t + l / 32. down = 0:
// gate/up bank, K = W, N = hidden, fragment ((g NB + nb) KS + s) 2 + which;
// down = 1: K = hidden, N = W, fragment (g KB + kb) NB + nb.
hipError_t launch_pack_mx(const uint16_t* src, uint8_t* dst, uint8_t* rec, int G, int K, int N, int down, int which,
                          int rec_dwords, hipStream_t s);
// MXFP8 sub-layer kernels (grid as launch_mlp): DENSE at W = 256 (two
// workgroups per CU) or 512; ROUTED and SHARED at W = 512 and 768
bool mlp_mx_supported(int mode, int W);
hipError_t launch_mlp_mx(int mode, int W, const MlpArgs& a, int tiles, int workers, hipStream_t s);
// hidden <= this many chunks of MLP_HC (the scale records of a tile sit in LDS)
constexpr int mx_max_chunks(int W) { return W == 768 ? 6 : 8; }
// dwords of one lane's scale record (a multiple of 4: the kernel moves it in
// 16-byte pieces)
constexpr int mx_rec_dwords(int W, int hidden) { return ((hidden / MLP_HC) * 3 * (W / 256) + 3) & ~3; }
// Mix / Revert through RowMap in one of its address forms (PermForm; see
// permute_kernel); forms other than PERM_ELEM need D/H % 8 == 0 and
// T*D/H % 32 == 0
enum PermForm { PERM_ELEM = 0, PERM_LANECOL = 1, PERM_CURSOR = 2 };
hipError_t launch_permute(const void* in, void* out, int B, int T, int D, int H, int elem_bytes,
                          int inverse, int form, hipStream_t s);

// RankMixer block (tmx_rankmixer.hip), bf16, H = T, D in {256, 512}:
//   part 0: out = S = rho(LN_1(TokenMixing(x) + x))
//   part 1: out = rho(LN_2(x + F_t(x)))               (x = S)
//   part 2: both in one kernel
//   part 3: experts only: the gates ReLU(x Wr_t) the FFN half uses, to
//           `gates` [B][T][E] fp32 (x = S)
// F_t is the token's FFN (E = 0) or its E ReLU-routed experts (D = 256,
// E in {16, 32}): W1 / W2 / b1 then hold the experts end to end (hidden =
// E * h_e), `wr` is the router ([T][D, E], 16x16x32 fragments, layout 1) and
// b2 the experts' second biases stacked twice ([T][2E, D], layout 2).
struct RmxArgs {
  int B, T, D, dh, hidden;
  int E, h_e;
  float eps;
  const uint16_t* x;       // [B, T, D]
  uint16_t* out;           // [B, T, D]
  const float* g1;         // LN_1 gain / bias [D]
  const float* be1;
  const float* g2;         // LN_2 gain / bias [D]
  const float* be2;
  const uint16_t* w1;      // W1 [T][D, hidden] packed with layout 2 (32x32x16 fragments)
  const uint16_t* w2;      // W2 [T][hidden, D] packed with layout 2
  const uint16_t* b1;      // [T][hidden] bf16
  const uint16_t* b2;      // [T][D] bf16 (experts: packed, see above)
  const uint16_t* wr;      // experts only: packed router
  float* gates;            // part 3 only
};
bool rmx_width_supported(int D);
int rmx_hidden_multiple(int D);   // the dense FFN's hidden must be a multiple (the kernel's chunk)
bool rmx_experts_supported(int D, int E, int h_e);
hipError_t launch_rmx(const RmxArgs& a, int part, hipStream_t s);

// Model front and back (tmx_io.hip), bf16: the tokenizer writes the tokens
// X [B, T, D] from the concatenated embeddings [B, F]; the head reads the
// stack's output Y [B, T, D] and writes one fp32 logit per sample.
struct IoArgs {
  int B, T, D, F, tok_hidden, head_hidden;
  const uint16_t* emb;       // [B, F]
  const int4* tok_pos;       // [T]: (column offset, K, first W1 fragment, 0)
  const uint16_t* tok_w1;    // position t's W1 [K_t, h] packed (32x32x16, layout 2) from tok_pos[t].z
  const uint16_t* tok_w2;    // [T] W2 [h, D] packed (32x32x16, layout 2)
  uint16_t* x_out;           // [B, T, D]
  const uint16_t* y;         // [B, T, D]
  const uint16_t* head_w1;   // W1 [D, h_head] packed (32x32x16, layout 2)
  const uint16_t* head_w2;   // [h_head] bf16
  float* logits;             // [B]
};
bool io_width_supported(int D);
bool io_tok_hidden_supported(int h);
bool io_head_hidden_supported(int h);
hipError_t launch_tokenize(const IoArgs& a, hipStream_t s);
hipError_t launch_head(const IoArgs& a, hipStream_t s);

// fp32 path
struct F32Args {
  int B, P, W, hidden, E, top_k, expert_hidden, shared_hidden;
  float alpha, eps;
  RowMap map;
  const float* x;
  const float* gain;
  const float* resid;      // nullable when route_only
  const float* extra;      // nullable
  float* out;              // nullable when route_only
  // dense
  const float* w_up;
  const float* w_gate;
  const float* w_down;
  // moe
  const float* w_router;
  const float* e_up;
  const float* e_gate;
  const float* e_down;
  const float* s_up;
  const float* s_gate;
  const float* s_down;
  int32_t* idx;            // nullable
  float* gate_out;         // nullable
  int route_only;
};
hipError_t launch_f32_sublayer(const F32Args& a, hipStream_t s);

}  // namespace tmx
