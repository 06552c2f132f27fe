/*
 * tmx.h -- C ABI of the MI355X (gfx950) TokenMixer-Large block-stack forward.
 *
 * The library computes the forward pass of the block stack described in
 * "TokenMixer-Large: Scaling Up Large Ranking Models in Industrial
 * Recommenders" (paper summary, sections 2.3-2.4, Eq. 9-21) and in the
 * tokenmixerlarge README's block diagram (Pre-Norm form):
 *
 *   for l = 1..L:   Hm     = Mix(Y_{l-1})                          (Eq. 9-11)
 *                   H_next = Hm + F_mix(RMSNorm(Hm))               (Eq. 12, Pre-Norm)
 *                   X_rev  = Revert(H_next)                        (Eq. 13-15)
 *                   Z_l    = Y_{l-1} + F_rev(RMSNorm(X_rev))       (Eq. 16, Pre-Norm)
 *                   Y_l    = Z_l + Y_{l-g} if g > 0, l % g == 0, l < L   (section 2.3.4)
 *
 * where every position p of a sub-layer owns its weights: F_p is a
 * per-token SwiGLU (Eq. 17-18) or a Sparse-Pertoken MoE (Eq. 19-21: top-k
 * softmax routing, gates alpha * pi, plus an always-on per-token shared
 * expert).  Mix sub-layer: P = H positions of width W = T*D/H.  Revert
 * sub-layer: P = T positions of width W = D.
 *
 * Conventions for every entry point:
 *  - Plain pointers and sizes only.  Tensors are dense row-major.
 *  - "device" pointers are HIP device allocations on the context's device;
 *    the caller owns them and the library never frees them.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Compute entry
 *    points only enqueue work (no host synchronisation, no host copies) and
 *    return before it has run; launch errors are reported as TMX_ERR_DEVICE.
 *  - All argument validation happens before anything is enqueued.  On any
 *    non-TMX_OK status nothing was enqueued and tmx_last_error() describes
 *    the failure.
 *  - A context is used by one host thread at a time.
 *  - Layers are numbered 0..L-1 (layer l here is the pages' block l+1).
 *
 * A context can instead hold a stack of RankMixer blocks (cfg.block =
 * TMX_BLOCK_RANKMIXER; fun-rec chapter 7.4.0 block equations, 7.4.1 token
 * mixing, 7.4.2 per-token FFN; the RankMixer reproduction README's per-token
 * FFN with biases), post-LN, no inter-residual:
 *
 *   for l = 1..L:   S   = LN_1(TokenMixing(X) + X)          (H = T, so the
 *                                                            mixed tensor has
 *                                                            the shape of X)
 *                   X   = LN_2(S + PFFN(S)),  PFFN_t(s) = GELU(s W1_t + b1_t) W2_t + b2_t
 *
 * LN is LayerNorm (biased variance, eps = cfg.eps, gain and bias), GELU the
 * erf form z * Phi(z) (erf evaluated to within 1.5e-7, Abramowitz & Stegun
 * 7.1.26).  Sub-layer 0 (TMX_MIX) is the token-mixing half, sub-layer
 * 1 (TMX_REVERT) the FFN half; S is rounded to the ctx dtype once.
 * With E > 0 each token's FFN is replaced by E ReLU-routed experts (fun-rec
 * chapter 7.4.3, the inference router of dense-train / sparse-infer):
 * G = ReLU(s Wr_t), PFFN_t(s) = sum_j G_j (GELU(s W1_tj + b1_tj) W2_tj + b2_tj),
 * a varying number of active experts per row; an expert that no row of a
 * 64-row tile activates is skipped for that tile.
 */
#ifndef TMX_H
#define TMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tmx_status {
  TMX_OK = 0,
  TMX_ERR_INVALID_ARG = 1, /* bad shape, index, pointer or size */
  TMX_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
  TMX_ERR_OOM = 3,         /* device allocation failed */
  TMX_ERR_DEVICE = 4,      /* a HIP runtime call or kernel launch failed */
  TMX_ERR_STATE = 5        /* e.g. forward before every weight was loaded */
} tmx_status;

/* TMX_MXFP8: bf16 activations and weights at the boundary, with the GEMM
 * operands of the per-token SwiGLUs quantised to MXFP8 inside the library
 * ("FP8 E4M3 post-training quantisation", TokenMixer-Large summary section
 * 2.5.2; read as E4M3 elements with one power-of-two scale per 32 values
 * along each GEMM's contraction axis): weights when they are loaded, the
 * normalised rows and the SwiGLU hidden in the kernel. Dense sub-layers of
 * width 256 or 512; MoE sub-layers of width 512 or 768, where the routed
 * and the shared experts run on MXFP8 operands and the router stays bf16
 * (section 2.4, Eq. 19-21). Hidden sizes a multiple of 128, at most 1024
 * (768 at width 768); other shapes give TMX_ERR_UNSUPPORTED. */
typedef enum tmx_dtype { TMX_F32 = 0, TMX_BF16 = 1, TMX_MXFP8 = 2 } tmx_dtype;

typedef enum tmx_sublayer { TMX_MIX = 0, TMX_REVERT = 1 } tmx_sublayer;

/* Block family of a context. */
typedef enum tmx_block { TMX_BLOCK_TOKENMIXER_LARGE = 0, TMX_BLOCK_RANKMIXER = 1 } tmx_block;

/* Weight kinds and their logical row-major layouts, with P and W of the
 * sub-layer (MIX: P = H, W = T*D/H; REVERT: P = T, W = D), h the dense
 * hidden of that sub-layer, E routed experts, h_e expert hidden, h_s
 * shared-expert hidden.  Row-vector convention y = x @ W (the RankMixer
 * reproduction guide's per-token banks W1 [T, D, kD], W2 [T, kD, D]). */
typedef enum tmx_weight_kind {
  TMX_W_NORM_GAIN = 0, /* [W]          RMSNorm gain, optional (default 1)  */
  TMX_W_UP = 1,        /* [P, W, h]    dense SwiGLU up       (Eq. 17-18)   */
  TMX_W_GATE = 2,      /* [P, W, h]    dense SwiGLU gate                   */
  TMX_W_DOWN = 3,      /* [P, h, W]    dense SwiGLU down                   */
  TMX_W_ROUTER = 4,    /* [P, W, E]    router, logits = x_hat @ Wr (Eq. 19) */
  TMX_W_EXP_UP = 5,    /* [P, E, W, h_e] routed experts (Eq. 19)           */
  TMX_W_EXP_GATE = 6,  /* [P, E, W, h_e]                                   */
  TMX_W_EXP_DOWN = 7,  /* [P, E, h_e, W]                                   */
  TMX_W_SH_UP = 8,     /* [P, W, h_s]  per-token shared expert (Eq. 20)    */
  TMX_W_SH_GATE = 9,   /* [P, W, h_s]                                      */
  TMX_W_SH_DOWN = 10,  /* [P, h_s, W]                                      */
  /* RankMixer contexts (P = T, W = D, h = hidden_rev): NORM_GAIN and
   * NORM_BIAS are LN_1's (sub-layer 0) or LN_2's (sub-layer 1); UP is W1
   * [T, D, h], DOWN is W2 [T, h, D] (sub-layer 1).  Gains default to 1,
   * biases to 0. */
  TMX_W_NORM_BIAS = 11, /* [W]          LayerNorm bias, optional            */
  TMX_W_BIAS_UP = 12,   /* [P, h]       b1 of the per-token FFN, optional   */
  TMX_W_BIAS_DOWN = 13, /* [P, W]       b2 of the per-token FFN, optional   */
  /* RankMixer ReLU-routed experts (E > 0, sub-layer 1): ROUTER [T, D, E] is
   * the inference router, EXP_UP [T, E, D, h_e] and EXP_DOWN [T, E, h_e, D]
   * the experts' W1 and W2. */
  TMX_W_EXP_BIAS_UP = 14,  /* [P, E, h_e] experts' b1, optional            */
  TMX_W_EXP_BIAS_DOWN = 15, /* [P, E, W]   experts' b2, optional           */
  /* The model's front and back (tmx_load_io_weights; F = sum of the group
   * widths, h the tokenizer hidden, h_head the head hidden):            */
  TMX_W_TOK_UP = 16,    /* [2F, h]   first layers of the tokenizer MLPs: the
                           global token's [F, h], then each group's [d_t, h]
                           in group order (Eq. 2-3)                        */
  TMX_W_TOK_DOWN = 17,  /* [T, h, D] second layers, token 0 (global) first  */
  TMX_W_HEAD_UP = 18,   /* [D, h_head] projection head, first layer         */
  TMX_W_HEAD_DOWN = 19  /* [h_head]  projection head, second layer (-> logit) */
} tmx_weight_kind;

/* Model configuration; the pages' problem statement (B, T, H, D, hidden, E,
 * top_k, L) plus the numerical knobs.  E = 0 selects the dense per-token
 * SwiGLU block; E > 0 the Sparse-Pertoken MoE in both sub-layers. */
typedef struct tmx_config {
  int32_t B_max;          /* largest batch a forward call may pass (>= 1)     */
  int32_t T;              /* tokens per sample (>= 1)                          */
  int32_t H;              /* heads / mixed tokens; D % H == 0 (RankMixer guide
                             section 5)                                        */
  int32_t D;              /* token width                                       */
  int32_t L;              /* number of blocks (>= 1)                           */
  int32_t hidden_mix;     /* dense: per-position hidden of the MIX sub-layer   */
  int32_t hidden_rev;     /* dense: per-position hidden of the REVERT sub-layer*/
  int32_t E;              /* routed experts per position (0 = dense)           */
  int32_t top_k;          /* experts chosen per row, 1 <= top_k <= E           */
  int32_t expert_hidden;  /* h_e                                               */
  int32_t shared_hidden;  /* h_s                                               */
  float alpha;            /* gate-value scaling (Eq. 21); 0 means E / top_k    */
  float eps;              /* RMSNorm (LayerNorm for RankMixer) epsilon (> 0)   */
  int32_t inter_residual_gap; /* g (section 2.3.4); 0 disables               */
  int32_t dtype;          /* tmx_dtype of activations and weights              */
  int32_t block;          /* tmx_block (0 = TokenMixer-Large)                  */
} tmx_config;

typedef struct tmx_ctx tmx_ctx;

/* Validate `cfg`, select `device` (hipSetDevice) and allocate the context:
 * weight storage for all L blocks and a workspace sized for B_max.
 * bf16 contexts additionally need D/H % 8 == 0, every sub-layer width W
 * (T*D/H for MIX, D for REVERT) one of 128, 256, 512, 768 and every hidden
 * size a multiple of 128; MoE contexts in bf16 need E % 16 == 0, E <= 64,
 * top_k <= 8 and B_max*T*D < 2^31 (the normalised-row workspace is
 * addressed with 32-bit byte offsets); TMX_ERR_UNSUPPORTED otherwise.
 * RankMixer contexts need H == T (the paper-strict token mixing; the
 * reproduction guide's section 5 makes any other H an error), hidden_mix ==
 * 0, inter_residual_gap == 0, and either hidden_rev >= 1 (dense) or E > 0
 * with hidden_rev == 0, top_k == 0 and expert_hidden >= 1
 * (TMX_ERR_INVALID_ARG otherwise); this build runs them in bf16 with D of
 * 256 or 512, D/H % 8 == 0 and hidden_rev a multiple of 128 (D = 256) or
 * 256 (D = 512), the experts at D = 256 with E of 16 or 32 and
 * expert_hidden % 128 == 0 (TMX_ERR_UNSUPPORTED otherwise).
 * On error *out is set to NULL and nothing stays allocated. */
tmx_status tmx_create(const tmx_config* cfg, int device, tmx_ctx** out);

/* Free everything the context owns (device memory, streams are the
 * caller's).  NULL is a no-op. */
tmx_status tmx_destroy(tmx_ctx* ctx);

/* Human-readable description of the last failure: of `ctx`, or of the
 * calling thread's last failed tmx_create when ctx is NULL.  The string is
 * owned by the library and valid until the next call on the same ctx. */
const char* tmx_last_error(const tmx_ctx* ctx);

/* Copy one weight bank (kind, layout as above, element type = ctx dtype)
 * of block `layer` (0..L-1), sub-layer `sublayer` (TMX_MIX / TMX_REVERT)
 * into the context and repack it into the kernels' fragment layout
 * (TMX_MXFP8: quantise it to E4M3 with per-32 E8M0 scales along the
 * contraction axis first).
 * `src` is a host or device pointer (detected with hipPointerGetAttributes);
 * the call copies and the caller keeps ownership.  `nbytes` must equal the
 * bank's exact size.  Dense contexts accept NORM_GAIN, UP, GATE, DOWN; MoE
 * contexts NORM_GAIN, ROUTER and the EXP_* / SH_* kinds; RankMixer contexts
 * NORM_GAIN and NORM_BIAS in both sub-layers and UP, DOWN, BIAS_UP,
 * BIAS_DOWN in sub-layer 1 (UP and DOWN are required); with E > 0 ROUTER,
 * EXP_UP, EXP_DOWN (required), EXP_BIAS_UP and EXP_BIAS_DOWN instead.  The call is
 * synchronous (it waits for `stream`); it is not meant for timed loops. */
tmx_status tmx_load_weights(tmx_ctx* ctx, int layer, int sublayer, int kind,
                            const void* src, size_t nbytes, void* stream);

/* Y_L = block stack applied to x_in.  x_in, x_out: device, [B, T, D]
 * row-major, ctx dtype, 16-byte aligned, not overlapping; 1 <= B <= B_max.
 * TMX_ERR_STATE if any required weight bank was never loaded. */
tmx_status tmx_block_stack_forward(tmx_ctx* ctx, const void* x_in, void* x_out,
                                   int B, void* stream);

/* The router of one MoE sub-layer (Eq. 19-21): x is that sub-layer's input
 * in block layout [B, T, D] (for TMX_MIX the Mix map is applied inside),
 * rows are normalised with the sub-layer's RMSNorm and rounded to the ctx
 * dtype, logits = x_hat @ Wr_p, pi = softmax over all E, and the top_k
 * experts under the key (-logit, expert index) are written in that order:
 * idx [B, P, top_k] int32 and gate [B, P, top_k] float32 = alpha * pi
 * (device pointers).  TMX_ERR_UNSUPPORTED on a dense or RankMixer context. */
tmx_status tmx_moe_route(tmx_ctx* ctx, int layer, int sublayer, const void* x,
                         int B, int32_t* idx, float* gate, void* stream);

/* tmx_sublayer_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, same arguments, same result, but a bf16 MoE
 * sub-layer keeps its workspace (normalised rows, routing table, bucket
 * lists, tile queues, expert outputs) in a static device array of 64 MiB
 * instead of the context's workspace; no call allocates or frees anything.
 * The array holds the workspace of B rows only up to its size:
 * TMX_ERR_INVALID_ARG names the largest B when a call needs more.  Dense,
 * fp32 and RankMixer sub-layers use no workspace and run as in
 * tmx_sublayer_forward.  Every call on one device shares that device's
 * array (it keeps the last call's contents; what must start at zero is
 * cleared by the kernels), so calls that overlap on one device -- on
 * different streams or from different contexts -- race. */
tmx_status tmx_sublayer_forward_noalloc(tmx_ctx* ctx, int layer, int sublayer,
                                        const void* x_in, const void* resid,
                                        const void* extra, void* x_out, int B,
                                        void* stream);

/* The normalised rows and the expert-first row lists of one MoE sub-layer
 * (RMSNorm, TokenMixer-Large summary section 2.3.3; MoEPermute, section
 * 2.5.1), for checks: x is the sub-layer's input in block layout [B, T, D]
 * (device); the sub-layer's router and bucket kernels run on it exactly as
 * in the forward, and what they wrote is copied out to each non-NULL
 * output (device pointers): xhat [P, B, W] bf16 (16-byte aligned), the rows
 * the experts consume; counts [P, E] int32 (rows routed to expert e at
 * position p); rows [P, B*top_k] int32, where position p's entries are
 * expert 0's, then expert 1's, ... (expert e's list starts at the exclusive
 * prefix sum of counts[p]) and each entry is b*top_k + slot, in ascending
 * order within a list.  Uses the context's workspace, so it must not
 * overlap a forward on another stream.  TMX_ERR_UNSUPPORTED unless the
 * context is a bf16 TokenMixer-Large MoE one. */
tmx_status tmx_moe_buckets(tmx_ctx* ctx, int layer, int sublayer, const void* x,
                           int B, void* xhat, int32_t* counts, int32_t* rows,
                           void* stream);

/* One sub-layer, for teacher-forced checks; runs the same kernels as the
 * forward.  All tensors are [B, T, D] in block layout (device).
 *   TMX_MIX:    x_out = Revert(Mix(x_in) + F_mix(RMSNorm(Mix(x_in))));
 *               `resid` and `extra` must be NULL.
 *   TMX_REVERT: x_out = resid + F_rev(RMSNorm(x_in)) [+ extra];
 *               `resid` is the block input, `extra` (nullable) the
 *               inter-residual term.
 * RankMixer contexts (`resid` and `extra` must be NULL):
 *   TMX_MIX:    x_out = S = LN_1(TokenMixing(x_in) + x_in);
 *   TMX_REVERT: x_out = LN_2(x_in + PFFN(x_in)), x_in being S.
 * The result is rounded once to the ctx dtype.  A chain of these calls
 * reproduces tmx_block_stack_forward bit for bit. */
tmx_status tmx_sublayer_forward(tmx_ctx* ctx, int layer, int sublayer,
                                const void* x_in, const void* resid,
                                const void* extra, void* x_out, int B,
                                void* stream);

/* The ReLU gates of one RankMixer block's experts (fun-rec chapter 7.4.3,
 * inference router): s is that block's FFN-half input S in block layout
 * [B, T, D] (device), gates [B, T, E] float32 (device) receives
 * ReLU(s_t Wr_t) per sample and token, as the block kernel applies them
 * (computed in fp32 from the bf16 operands, carried to 16 significant
 * bits).  TMX_ERR_UNSUPPORTED unless the context is a RankMixer one with
 * E > 0; TMX_ERR_STATE if that layer's router was never loaded. */
tmx_status tmx_relu_route(tmx_ctx* ctx, int layer, const void* s, int B, float* gates, void* stream);

/* Address forms of the Mix / Revert map that tmx_debug_permute can run. */
typedef enum tmx_perm_form {
  TMX_PERM_ELEMENT = 0, /* one offset computation per element (fp32 path; the
                           fused MLP's row I/O where a lane's columns change
                           from unit to unit, W = 768)                      */
  TMX_PERM_LANECOL = 1, /* the fused MLP's row I/O: 8-column units of whole
                           rows, a lane's column part computed once         */
  TMX_PERM_CURSOR = 2   /* the router's row loads: a row's 8-column runs at a
                           stride of 32 columns through the column cursor   */
} tmx_perm_form;

/* Apply Mix (inverse = 0: out [B, H, T*D/H]) or Revert (inverse = 1:
 * in [B, H, T*D/H] -> out [B, T, D]) (TokenMixer-Large Eq. 9-11, 13-15):
 * bit-exact data movement through the library's single Mix / Revert address
 * map, in the address form `form` (tmx_perm_form) -- the device functions
 * and the unit-to-lane assignment the sub-layer kernels run.  in and out
 * are device buffers of the ctx dtype, not overlapping; forms 1 and 2 need
 * 16-byte aligned buffers, D/H % 8 == 0 and T*D/H % 32 == 0
 * (TMX_ERR_UNSUPPORTED otherwise). */
tmx_status tmx_debug_permute(tmx_ctx* ctx, const void* in, void* out, int B,
                             int inverse, int form, void* stream);

/* ---- The model around the stack: tokenizer front and mean-pool head ----
 * TokenMixer-Large summary section 2.2 (Eq. 1-4) and section 2.1; the
 * tokenmixerlarge README's block diagram (group MLPs + global MLP -> tokens;
 * mean-pool over tokens -> projection head -> logit).  The tokenizer maps
 * the concatenated feature embeddings emb [B, F] (F = sum of the T - 1
 * semantic group widths d_t, group t in columns [sum_{u<t} d_u, +d_t)) to
 * the tokens X [B, T, D]: X[:, t] = MLP_t(group t's columns) for t >= 1
 * (Eq. 2) and the global token X[:, 0] = MLP_g(all F columns) (Eq. 3-4).
 * The head averages the T tokens of Y [B, T, D] and maps the mean to one
 * logit per sample.  Every MLP is v -> ReLU(v W1) W2 without biases.  bf16:
 * the hidden ReLU outputs, the tokens and the pooled mean are rounded to
 * bf16 once each; GEMMs accumulate in fp32; the logit is fp32. */

/* Declare the tokenizer and head of a bf16 (or MXFP8) context once:
 * n_groups must be T - 1, group widths multiples of 32, tok_hidden in
 * {128, 256, 512, 768}, head_hidden in {128, 256, 512}, D in {128, 256, 512,
 * 768} (TMX_ERR_UNSUPPORTED otherwise).  Allocates their weight storage
 * and two [B_max, T, D] buffers for tmx_model_forward.  TMX_ERR_STATE if
 * called twice. */
tmx_status tmx_set_model_io(tmx_ctx* ctx, const int32_t* group_widths, int n_groups,
                            int tok_hidden, int head_hidden);

/* Copy one tokenizer or head bank (TMX_W_TOK_UP .. TMX_W_HEAD_DOWN, row-major
 * bf16, host or device `src`, exact `nbytes`) into the context and repack it
 * into MFMA fragments.  Synchronous.  TMX_ERR_STATE before tmx_set_model_io. */
tmx_status tmx_load_io_weights(tmx_ctx* ctx, int kind, const void* src, size_t nbytes,
                               void* stream);

/* X = tokenizer(emb): emb [B, F] bf16, x_out [B, T, D] bf16, device, 16-byte
 * aligned, not overlapping; 1 <= B <= B_max.  TMX_ERR_STATE unless both
 * tokenizer banks are loaded. */
tmx_status tmx_tokenize(tmx_ctx* ctx, const void* emb, void* x_out, int B, void* stream);

/* logits[b] = head(mean over t of y[b, t, :]): y [B, T, D] bf16 (device,
 * 16-byte aligned), logits [B] float32 (device).  TMX_ERR_STATE unless both
 * head banks are loaded. */
tmx_status tmx_head(tmx_ctx* ctx, const void* y, float* logits, int B, void* stream);

/* The whole model: logits = head(block stack(tokenizer(emb))), through the
 * context's own token buffers; same arguments as tmx_tokenize / tmx_head.
 * TMX_ERR_STATE unless every bank of the stack, tokenizer and head is
 * loaded. */
tmx_status tmx_model_forward(tmx_ctx* ctx, const void* emb, float* logits, int B, void* stream);

/* Kernels of the library, as counted by tmx_kernel_times. */
typedef enum tmx_kernel_kind {
  TMX_KERNEL_MLP_DENSE = 0,  /* fused per-position SwiGLU sub-layer (Eq. 12-18)  */
  TMX_KERNEL_MLP_ROUTED = 1, /* grouped routed experts (section 2.5.1 GroupedFFN) */
  TMX_KERNEL_MLP_SHARED = 2, /* shared expert + gated combine (Eq. 20-21)        */
  TMX_KERNEL_ROUTER = 3,     /* RMSNorm + router + top-k (Eq. 19, 21)            */
  TMX_KERNEL_BUCKET = 4,     /* expert-first row lists (section 2.5.1 MoEPermute) */
  TMX_KERNEL_RMX_BLOCK = 5,  /* RankMixer block                                  */
  TMX_KERNEL_F32 = 6,        /* fp32 sub-layer                                   */
  TMX_KERNEL_TOKENIZE = 7,   /* semantic group-wise tokenizer (Eq. 2-4)          */
  TMX_KERNEL_HEAD = 8,       /* mean pool + projection head (section 2.1)       */
  TMX_KERNEL_KINDS = 9
} tmx_kernel_kind;

/* Measurement: with enable = 1 every kernel the context enqueues from then
 * on is bracketed by a pair of HIP events recorded on its launch stream
 * (events are created on first use and reused); enable = 0 stops that. */
tmx_status tmx_set_kernel_timing(tmx_ctx* ctx, int enable);

/* Waits for every bracketed launch, then writes, for the first n kernel kinds
 * (tmx_kernel_kind), the summed event-timed duration in milliseconds and the
 * number of launches since the previous call (host arrays ms[n] and
 * launches[n]), and resets both.  Synchronises with the recorded streams;
 * not for use inside a captured or timed region. */
tmx_status tmx_kernel_times(tmx_ctx* ctx, double* ms, long long* launches, int n);

#ifdef __cplusplus
}
#endif
#endif /* TMX_H */
