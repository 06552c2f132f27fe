/* Drives the host side of the C ABI (validation, error reporting, NULL
 * handling) in a build of the host library instrumented with AddressSanitizer
 * and UndefinedBehaviorSanitizer. No GPU is needed: every call returns before
 * a launch, and creating a valid context reports TMX_ERR_DEVICE when no
 * device is present. Prints "abi-sanitize ok <checks>" and exits 0, or names
 * the first failed check and exits 1; a sanitizer report aborts the run. */
#include <stdio.h>
#include <string.h>

#include "tmx.h"

static int checks = 0;

#define EXPECT(cond, what)                                       \
  do {                                                           \
    ++checks;                                                    \
    if (!(cond)) {                                               \
      fprintf(stderr, "abi-sanitize: failed check: %s\n", what); \
      return 1;                                                  \
    }                                                            \
  } while (0)

static tmx_config base(void) {
  tmx_config c;
  memset(&c, 0, sizeof c);
  c.B_max = 16; c.T = 4; c.H = 4; c.D = 32; c.L = 1;
  c.hidden_mix = 64; c.hidden_rev = 64;
  c.eps = 1e-6f; c.inter_residual_gap = 2; c.dtype = TMX_F32;
  return c;
}

static int create_status(tmx_config c) {
  tmx_ctx* h = (tmx_ctx*)0x1;
  int st = tmx_create(&c, 0, &h);
  if (h != NULL) return -1;
  const char* m = tmx_last_error(NULL);
  if (!m || !m[0]) return -2;
  return st;
}

int main(void) {
  tmx_ctx* h = NULL;
  EXPECT(tmx_create(NULL, 0, &h) == TMX_ERR_INVALID_ARG && h == NULL, "NULL cfg");
  tmx_config c = base();
  EXPECT(tmx_create(&c, 0, NULL) == TMX_ERR_INVALID_ARG, "NULL out");

  struct {
    const char* what;
    int field;
    int value;
    int want;
  } cases[] = {
      {"D % H", 0, 30, TMX_ERR_INVALID_ARG},        {"T = 0", 1, 0, TMX_ERR_INVALID_ARG},
      {"H = 0", 2, 0, TMX_ERR_INVALID_ARG},         {"L = 0", 3, 0, TMX_ERR_INVALID_ARG},
      {"B_max = 0", 4, 0, TMX_ERR_INVALID_ARG},     {"gap < 0", 5, -1, TMX_ERR_INVALID_ARG},
      {"hidden_mix = 0", 6, 0, TMX_ERR_INVALID_ARG}, {"dtype 7", 7, 7, TMX_ERR_INVALID_ARG},
      {"block 2", 8, 2, TMX_ERR_INVALID_ARG},       {"E < 0", 9, -1, TMX_ERR_INVALID_ARG},
  };
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    c = base();
    switch (cases[i].field) {
      case 0: c.D = cases[i].value; break;
      case 1: c.T = cases[i].value; break;
      case 2: c.H = cases[i].value; break;
      case 3: c.L = cases[i].value; break;
      case 4: c.B_max = cases[i].value; break;
      case 5: c.inter_residual_gap = cases[i].value; break;
      case 6: c.hidden_mix = cases[i].value; break;
      case 7: c.dtype = cases[i].value; break;
      case 8: c.block = cases[i].value; break;
      default: c.E = cases[i].value; break;
    }
    EXPECT(create_status(c) == cases[i].want, cases[i].what);
  }
  /* MXFP8 with H = 0 or H not dividing D: a shape error, never a division */
  c = base(); c.dtype = TMX_MXFP8; c.D = 256; c.T = 16; c.H = 0; c.hidden_mix = 256; c.hidden_rev = 256;
  EXPECT(create_status(c) == TMX_ERR_INVALID_ARG, "MXFP8 H = 0");
  c.H = 7;
  EXPECT(create_status(c) == TMX_ERR_INVALID_ARG, "MXFP8 D % H");
  /* MoE shape errors */
  c = base(); c.E = 4; c.top_k = 5; c.expert_hidden = 8; c.shared_hidden = 8;
  EXPECT(create_status(c) == TMX_ERR_INVALID_ARG, "top_k > E");
  c.top_k = 2; c.alpha = -1.f;
  EXPECT(create_status(c) == TMX_ERR_INVALID_ARG, "alpha < 0");
  c = base(); c.eps = 0.f;
  EXPECT(create_status(c) == TMX_ERR_INVALID_ARG, "eps = 0");
  /* capability limits of the bf16 path */
  c = base(); c.dtype = TMX_BF16; c.D = 96;
  EXPECT(create_status(c) == TMX_ERR_UNSUPPORTED, "bf16 W = 96");
  /* a valid configuration without a device */
  c = base();
  int st = create_status(c);
  EXPECT(st == TMX_ERR_DEVICE || st == TMX_OK, "valid config: device error or success");

  /* every entry point with a NULL context */
  EXPECT(tmx_destroy(NULL) == TMX_OK, "destroy NULL");
  EXPECT(tmx_load_weights(NULL, 0, 0, 1, NULL, 0, NULL) == TMX_ERR_INVALID_ARG, "load NULL");
  EXPECT(tmx_block_stack_forward(NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG, "forward NULL");
  EXPECT(tmx_moe_route(NULL, 0, 0, NULL, 1, NULL, NULL, NULL) == TMX_ERR_INVALID_ARG, "route NULL");
  EXPECT(tmx_moe_buckets(NULL, 0, 0, NULL, 1, NULL, NULL, NULL, NULL) == TMX_ERR_INVALID_ARG, "buckets NULL");
  EXPECT(tmx_sublayer_forward(NULL, 0, 0, NULL, NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG, "sublayer NULL");
  EXPECT(tmx_sublayer_forward_noalloc(NULL, 0, 0, NULL, NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG,
         "sublayer noalloc NULL");
  EXPECT(tmx_relu_route(NULL, 0, NULL, 1, NULL, NULL) == TMX_ERR_INVALID_ARG, "relu route NULL");
  EXPECT(tmx_debug_permute(NULL, NULL, NULL, 1, 0, 0, NULL) == TMX_ERR_INVALID_ARG, "permute NULL");
  EXPECT(tmx_set_kernel_timing(NULL, 1) == TMX_ERR_INVALID_ARG, "timing NULL");
  EXPECT(tmx_kernel_times(NULL, NULL, NULL, 0) == TMX_ERR_INVALID_ARG, "times NULL");
  EXPECT(tmx_set_model_io(NULL, NULL, 0, 128, 128) == TMX_ERR_INVALID_ARG, "set model io NULL");
  EXPECT(tmx_load_io_weights(NULL, TMX_W_TOK_UP, NULL, 0, NULL) == TMX_ERR_INVALID_ARG, "io weights NULL");
  EXPECT(tmx_tokenize(NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG, "tokenize NULL");
  EXPECT(tmx_head(NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG, "head NULL");
  EXPECT(tmx_model_forward(NULL, NULL, NULL, 1, NULL) == TMX_ERR_INVALID_ARG, "model forward NULL");
  EXPECT(tmx_last_error(NULL) != NULL, "last error");
  printf("abi-sanitize ok %d\n", checks);
  return 0;
}
