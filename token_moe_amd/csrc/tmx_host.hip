// tmx_host.hip -- the C ABI (include/tmx.h): validation, weight storage and
// repacking, workspace, and the launch sequence of the block-stack forward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tmx.h"
#include "tmx_internal.h"

using namespace tmx;

namespace {

constexpr int NKINDS = 16;
thread_local std::string g_create_error;

// Scratch of tmx_sublayer_forward_noalloc: the MoE workspace of one
// sub-layer call, for callers that cannot allocate. Each device holds its
// own copy of the array for the life of the process. Host code never uses
// the array's name as an address: tmx_create looks up each device's copy
// with hipGetSymbolAddress (that device current) and keeps the pointer.
constexpr size_t TMX_SCRATCH_BYTES = size_t(64) << 20;
constexpr int TMX_SCRATCH_DEVICES = 64;
static __device__ __align__(256) uint8_t scratch[TMX_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[TMX_SCRATCH_DEVICES] = {};
hipError_t g_scratch_err[TMX_SCRATCH_DEVICES] = {};

// once per device, with that device current
void setup_scratch(int device) {
  if (device < 0 || device >= TMX_SCRATCH_DEVICES) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    g_scratch_err[device] = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return;
  }
  g_scratch_ptr[device] = p;
}

struct Bank {
  void* ptr = nullptr;    // device storage (packed for bf16 matrices, fp32 for gains)
  size_t elems = 0;       // logical element count
  bool loaded = false;
};

// The device workspace of a bf16 MoE sub-layer: everything its kernels
// write besides the output. One region, carved by carve_moe_ws(); the
// context's own region is laid out for B_max, the static scratch of
// tmx_sublayer_forward_noalloc for the call's B.
struct MoeWs {
  uint16_t* xhat = nullptr;   // [P][B][W] normalised rows (largest sub-layer)
  int32_t* idx = nullptr;     // [B][P][k]
  float* gate = nullptr;      // [B][P][k]
  int* rows = nullptr;        // [P][B*k] expert-first row lists
  int4* tiles = nullptr;      // [P][max_tiles] (expert, start, count, 0)
  int* ntiles = nullptr;      // [P]
  int* counts = nullptr;      // [P][E]
  int* qhead = nullptr;       // [8] routed-MLP tile queues (zeroed by the bucket kernel)
  int* hist = nullptr;        // [P][chunks][E] router choices per row chunk (128 rows; sized for 64)
  uint16_t* part = nullptr;   // [B][P][k][W] gated expert outputs, bf16
  uint8_t* xq8 = nullptr;     // MXFP8 MoE only: x_hat's E4M3 codes [P][B][W], then
                              // its exponents [P][B][W/32] (the router's output
                              // that the expert kernels read instead of xhat)
};

}  // namespace

struct tmx_ctx {
  tmx_config cfg{};
  int device = 0;
  int workers = 0;              // persistent-kernel grid: compute units on the device
  float alpha = 0.f;
  std::vector<Bank> banks;      // [L][2][NKINDS]
  // workspace
  void* act[3] = {nullptr, nullptr, nullptr};  // [B_max, T, D] each
  void* xrev = nullptr;                        // [B_max, T, D]
  MoeWs ws;                                    // bf16 MoE workspace, laid out for B_max
  // model front and back (tmx_set_model_io)
  struct Io {
    bool set = false;
    int F = 0, h = 0, hh = 0;
    std::vector<int> widths;                   // T - 1 group widths
    int4* pos = nullptr;                       // device [T]: (column offset, K, first W1 fragment, 0)
    uint16_t* w1 = nullptr;                    // packed W1 of every position
    uint16_t* w2 = nullptr;                    // packed [T] W2
    uint16_t* hw1 = nullptr;                   // packed head W1
    uint16_t* hw2 = nullptr;                   // head w2 [hh] bf16
    void* xbuf = nullptr;                      // tmx_model_forward: tokens [B_max, T, D]
    void* ybuf = nullptr;                      // tmx_model_forward: stack output
    bool loaded[4] = {};
  } io;
  std::vector<void*> allocs;
  std::string err;
  // per-kernel timing (tmx_set_kernel_timing): an event pair around every
  // launch while enabled, harvested by tmx_kernel_times
  struct Timed {
    int kind;
    hipEvent_t start, end;
  };
  bool timing = false;
  std::vector<Timed> pending;
  std::vector<hipEvent_t> event_pool;
  double kernel_ms[TMX_KERNEL_KINDS] = {};
  long long kernel_launches[TMX_KERNEL_KINDS] = {};
};

namespace {

tmx_status fail(tmx_ctx* c, tmx_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c)
    c->err = buf;
  else
    g_create_error = buf;
  return s;
}

size_t esize(const tmx_config& c) { return c.dtype == TMX_F32 ? 4 : 2; }   // MXFP8: bf16 activations
int positions(const tmx_config& c, int sub) { return sub == TMX_MIX ? c.H : c.T; }
int width(const tmx_config& c, int sub) { return sub == TMX_MIX ? c.T * (c.D / c.H) : c.D; }
int dense_hidden(const tmx_config& c, int sub) { return sub == TMX_MIX ? c.hidden_mix : c.hidden_rev; }
bool is_moe(const tmx_config& c) { return c.E > 0; }
bool is_rmx(const tmx_config& c) { return c.block == TMX_BLOCK_RANKMIXER; }
bool is_norm(int kind) { return kind == TMX_W_NORM_GAIN || kind == TMX_W_NORM_BIAS; }
// kinds a context may go without: gains default to 1, biases to 0
bool is_bias(int kind) {
  return kind == TMX_W_BIAS_UP || kind == TMX_W_BIAS_DOWN || kind == TMX_W_EXP_BIAS_UP || kind == TMX_W_EXP_BIAS_DOWN;
}

// logical [G, K, N] view of a matrix bank; returns false for non-matrix kinds
bool bank_dims(const tmx_config& c, int sub, int kind, int64_t* G, int* K, int* N) {
  const int P = positions(c, sub), W = width(c, sub);
  switch (kind) {
    case TMX_W_UP: case TMX_W_GATE: *G = P; *K = W; *N = dense_hidden(c, sub); return true;
    case TMX_W_DOWN: *G = P; *K = dense_hidden(c, sub); *N = W; return true;
    case TMX_W_ROUTER: *G = P; *K = W; *N = c.E; return true;
    case TMX_W_EXP_UP: case TMX_W_EXP_GATE: *G = (int64_t)P * c.E; *K = W; *N = c.expert_hidden; return true;
    case TMX_W_EXP_DOWN: *G = (int64_t)P * c.E; *K = c.expert_hidden; *N = W; return true;
    case TMX_W_SH_UP: case TMX_W_SH_GATE: *G = P; *K = W; *N = c.shared_hidden; return true;
    case TMX_W_SH_DOWN: *G = P; *K = c.shared_hidden; *N = W; return true;
    default: return false;
  }
}

bool kind_applies(const tmx_config& c, int sub, int kind) {
  if (is_rmx(c)) {
    if (is_norm(kind)) return true;
    if (sub != TMX_REVERT) return false;
    if (is_moe(c))
      return kind == TMX_W_ROUTER || kind == TMX_W_EXP_UP || kind == TMX_W_EXP_DOWN || kind == TMX_W_EXP_BIAS_UP ||
             kind == TMX_W_EXP_BIAS_DOWN;
    return kind == TMX_W_UP || kind == TMX_W_DOWN || kind == TMX_W_BIAS_UP || kind == TMX_W_BIAS_DOWN;
  }
  if (kind == TMX_W_NORM_GAIN) return true;
  if (is_moe(c)) return kind >= TMX_W_ROUTER && kind <= TMX_W_SH_DOWN;
  return kind >= TMX_W_UP && kind <= TMX_W_DOWN;
}

size_t kind_elems(const tmx_config& c, int sub, int kind) {
  if (is_norm(kind)) return (size_t)width(c, sub);
  if (kind == TMX_W_BIAS_UP) return (size_t)positions(c, sub) * dense_hidden(c, sub);
  if (kind == TMX_W_BIAS_DOWN) return (size_t)positions(c, sub) * width(c, sub);
  if (kind == TMX_W_EXP_BIAS_UP) return (size_t)positions(c, sub) * c.E * c.expert_hidden;
  if (kind == TMX_W_EXP_BIAS_DOWN) return (size_t)positions(c, sub) * c.E * width(c, sub);
  int64_t G;
  int K, N;
  if (!bank_dims(c, sub, kind, &G, &K, &N)) return 0;
  return (size_t)G * K * N;
}

Bank& bank(tmx_ctx* c, int layer, int sub, int kind) {
  return c->banks[((size_t)layer * 2 + sub) * NKINDS + kind];
}

// storage of a bank: gate and up share one interleaved fragment buffer in bf16
Bank& storage(tmx_ctx* c, int layer, int sub, int kind) {
  if (c->cfg.dtype != TMX_F32 && !is_rmx(c->cfg)) {
    if (kind == TMX_W_UP) kind = TMX_W_GATE;
    if (kind == TMX_W_EXP_UP) kind = TMX_W_EXP_GATE;
    if (kind == TMX_W_SH_UP) kind = TMX_W_SH_GATE;
  }
  return bank(c, layer, sub, kind);
}

// MXFP8: the gate kind of a matrix family (dense, routed experts, shared
// expert) -- its buffer holds the family's gate|up codes, then the scale
// records of gate, up and down -- or -1 for kinds kept in bf16 (the router)
int mx_gate_kind(int kind) {
  switch (kind) {
    case TMX_W_UP: case TMX_W_GATE: case TMX_W_DOWN: return TMX_W_GATE;
    case TMX_W_EXP_UP: case TMX_W_EXP_GATE: case TMX_W_EXP_DOWN: return TMX_W_EXP_GATE;
    case TMX_W_SH_UP: case TMX_W_SH_GATE: case TMX_W_SH_DOWN: return TMX_W_SH_GATE;
    default: return -1;
  }
}
// dwords per lane of a family's scale records, and the records' bytes
int mx_rec(const tmx_config& c, int sub, int gate_kind) {
  int64_t G;
  int K, N;
  bank_dims(c, sub, gate_kind, &G, &K, &N);
  return mx_rec_dwords(K, N);
}
size_t mx_rec_bytes(const tmx_config& c, int sub, int gate_kind) {
  int64_t G;
  int K, N;
  bank_dims(c, sub, gate_kind, &G, &K, &N);
  return (size_t)G * 4 * 64 * mx_rec(c, sub, gate_kind) * 4;
}

void release(tmx_ctx* c) {
  for (void* p : c->allocs) (void)hipFree(p);
  c->allocs.clear();
}

tmx_status dev_alloc(tmx_ctx* c, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  if (bytes == 0) return TMX_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(c, e == hipErrorOutOfMemory ? TMX_ERR_OOM : TMX_ERR_DEVICE, "hipMalloc(%zu bytes) for %s: %s",
                bytes, what, hipGetErrorString(e));
  }
  c->allocs.push_back(*p);
  return TMX_OK;
}

tmx_status check_launch(tmx_ctx* c, hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return TMX_OK;
}

hipEvent_t take_event(tmx_ctx* c) {
  if (!c->event_pool.empty()) {
    hipEvent_t e = c->event_pool.back();
    c->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

// launch() enqueues one kernel; with timing on, HIP events on the same
// stream bracket it (kernel kind `kind`, tmx_kernel_kind)
template <class F>
tmx_status launch_timed(tmx_ctx* c, int kind, hipStream_t st, const char* what, F&& launch) {
  if (!c->timing) return check_launch(c, launch(), what);
  hipEvent_t a = take_event(c), b = take_event(c);
  if (a) (void)hipEventRecord(a, st);
  tmx_status s = check_launch(c, launch(), what);
  if (a && b && hipEventRecord(b, st) == hipSuccess)
    c->pending.push_back({kind, a, b});
  else {
    if (a) c->event_pool.push_back(a);
    if (b) c->event_pool.push_back(b);
  }
  return s;
}

tmx_status validate_config(const tmx_config* cfg) {
  if (!cfg) return fail(nullptr, TMX_ERR_INVALID_ARG, "cfg is NULL");
  const tmx_config& c = *cfg;
  if (c.dtype != TMX_F32 && c.dtype != TMX_BF16 && c.dtype != TMX_MXFP8)
    return fail(nullptr, TMX_ERR_INVALID_ARG, "dtype must be TMX_F32 (0), TMX_BF16 (1) or TMX_MXFP8 (2), got %d",
                c.dtype);
  if (c.B_max < 1 || c.T < 1 || c.H < 1 || c.D < 1 || c.L < 1)
    return fail(nullptr, TMX_ERR_INVALID_ARG, "B_max, T, H, D, L must be >= 1 (got %d, %d, %d, %d, %d)", c.B_max,
                c.T, c.H, c.D, c.L);
  if (c.D % c.H != 0) return fail(nullptr, TMX_ERR_INVALID_ARG, "D (%d) must be divisible by H (%d)", c.D, c.H);
  if (!(c.eps > 0.f)) return fail(nullptr, TMX_ERR_INVALID_ARG, "eps must be > 0");
  if (c.inter_residual_gap < 0) return fail(nullptr, TMX_ERR_INVALID_ARG, "inter_residual_gap must be >= 0");
  if (c.E < 0) return fail(nullptr, TMX_ERR_INVALID_ARG, "E must be >= 0");
  if (c.block != TMX_BLOCK_TOKENMIXER_LARGE && c.block != TMX_BLOCK_RANKMIXER)
    return fail(nullptr, TMX_ERR_INVALID_ARG, "block must be 0 (TokenMixer-Large) or 1 (RankMixer), got %d", c.block);
  if (is_rmx(c)) {
    if (c.H != c.T)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "RankMixer token mixing needs H == T (got H %d, T %d)", c.H, c.T);
    if (c.hidden_mix != 0 || c.inter_residual_gap != 0)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "RankMixer blocks take hidden_mix = 0 and inter_residual_gap = 0");
    if (c.E == 0 && c.hidden_rev < 1) return fail(nullptr, TMX_ERR_INVALID_ARG, "RankMixer needs hidden_rev (kD) >= 1");
    if (c.E > 0 && (c.hidden_rev != 0 || c.top_k != 0 || c.expert_hidden < 1))
      return fail(nullptr, TMX_ERR_INVALID_ARG,
                  "RankMixer ReLU-routed experts take hidden_rev = 0, top_k = 0 (the count of active experts varies) "
                  "and expert_hidden >= 1");
    if (c.dtype != TMX_BF16) return fail(nullptr, TMX_ERR_UNSUPPORTED, "RankMixer blocks run in bf16 in this build");
    if (!rmx_width_supported(c.D))
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "RankMixer path supports D = 256 or 512, got %d", c.D);
    if ((c.D / c.H) % 8 != 0)
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "RankMixer path needs D/H %% 8 == 0, got %d", c.D / c.H);
    if (c.E == 0 && c.hidden_rev % rmx_hidden_multiple(c.D) != 0)
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "RankMixer path at D = %d needs hidden_rev %% %d == 0, got %d", c.D,
                  rmx_hidden_multiple(c.D), c.hidden_rev);
    if (c.E > 0 && !rmx_experts_supported(c.D, c.E, c.expert_hidden))
      return fail(nullptr, TMX_ERR_UNSUPPORTED,
                  "RankMixer experts need D = 256, E of 16 or 32 and expert_hidden %% 128 == 0 (got D %d, E %d, "
                  "h_e %d)", c.D, c.E, c.expert_hidden);
    if ((int64_t)c.B_max * c.T * c.D > (int64_t)1 << 40)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "B_max*T*D too large");
    return TMX_OK;
  }
  if (c.E == 0) {
    if (c.hidden_mix < 1 || c.hidden_rev < 1)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "dense config needs hidden_mix, hidden_rev >= 1");
  } else {
    if (c.top_k < 1 || c.top_k > c.E)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "need 1 <= top_k <= E (top_k %d, E %d)", c.top_k, c.E);
    if (c.expert_hidden < 1 || c.shared_hidden < 1)
      return fail(nullptr, TMX_ERR_INVALID_ARG, "MoE config needs expert_hidden, shared_hidden >= 1");
    if (c.alpha < 0.f) return fail(nullptr, TMX_ERR_INVALID_ARG, "alpha must be >= 0");
  }
  const int64_t act = (int64_t)c.B_max * c.T * c.D;
  if (act > (int64_t)1 << 40) return fail(nullptr, TMX_ERR_INVALID_ARG, "B_max*T*D too large");
  if (c.dtype == TMX_MXFP8) {
    // (bf16 activations: the bf16 checks below apply as well)
    for (int sub = 0; sub < 2; ++sub) {
      const int W = width(c, sub);
      if (!mlp_mx_supported(c.E > 0 ? MLP_ROUTED : MLP_DENSE, W))
        return fail(nullptr, TMX_ERR_UNSUPPORTED,
                    "MXFP8 path supports sub-layer widths 256 and 512 (dense) or 512 and 768 (MoE), got %d", W);
      const int hs[2] = {c.E ? c.expert_hidden : dense_hidden(c, sub), c.E ? c.shared_hidden : MLP_HC};
      for (int h : hs)
        if (h % MLP_HC != 0 || h > mx_max_chunks(W) * MLP_HC)
          return fail(nullptr, TMX_ERR_UNSUPPORTED,
                      "MXFP8 path needs hidden %% %d == 0 and hidden <= %d at width %d, got %d", MLP_HC,
                      mx_max_chunks(W) * MLP_HC, W, h);
    }
  }

  const int dh = c.D / c.H;
  if (c.dtype == TMX_BF16 || c.dtype == TMX_MXFP8) {
    if (dh % 8 != 0)
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "bf16 path needs D/H %% 8 == 0 (16-byte Mix segments), got %d", dh);
    for (int sub = 0; sub < 2; ++sub) {
      const int W = width(c, sub);
      if (!mlp_width_supported(W))
        return fail(nullptr, TMX_ERR_UNSUPPORTED, "bf16 path supports sub-layer widths 128, 256, 512, 768; got %d",
                    W);
      const int hs[2] = {c.E ? c.expert_hidden : dense_hidden(c, sub), c.E ? c.shared_hidden : MLP_HC};
      for (int h : hs)
        if (h % MLP_HC != 0)
          return fail(nullptr, TMX_ERR_UNSUPPORTED, "bf16 path needs hidden sizes %% %d == 0, got %d", MLP_HC, h);
    }
    if (c.E > 0 && (c.E % 16 != 0 || c.E > 64))
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "bf16 MoE needs E %% 16 == 0 and E <= 64, got %d", c.E);
    if (c.E > 0 && c.top_k > 8) return fail(nullptr, TMX_ERR_UNSUPPORTED, "bf16 MoE needs top_k <= 8");
    if (c.E > 0 && act >= (int64_t)1 << 31)
      return fail(nullptr, TMX_ERR_UNSUPPORTED,
                  "bf16 MoE needs B_max*T*D < 2^31 (the x_hat workspace is addressed with 32-bit byte offsets)");
  } else if (c.dtype == TMX_F32) {
    if (c.E > 256 || c.top_k > 64) return fail(nullptr, TMX_ERR_UNSUPPORTED, "fp32 MoE needs E <= 256, top_k <= 64");
    const int hmax = std::max({c.hidden_mix, c.hidden_rev, c.expert_hidden, c.shared_hidden});
    const int Wmax = std::max(width(c, 0), width(c, 1));
    if ((2LL * Wmax + hmax + std::max(c.E, 1) + 2) * 4 > 65536)
      return fail(nullptr, TMX_ERR_UNSUPPORTED, "fp32 path needs (2W + hidden + E) * 4 bytes <= 64 KiB of LDS");
  }
  return TMX_OK;
}

// rows per routed bucket tile: the wide routed kernel's where it applies
int moe_bm(const tmx_config& c, int sub) {
  const int wide = c.dtype == TMX_BF16     ? routed_wide_rows(width(c, sub), c.expert_hidden)
                   : c.dtype == TMX_MXFP8 ? routed_wide_mx_rows(width(c, sub), c.expert_hidden)
                                          : 0;
  return wide > 0 ? wide : mlp_bm(MLP_ROUTED, width(c, sub));
}
int moe_max_tiles(const tmx_config& c, int sub, int B) {
  const int bm = moe_bm(c, sub);
  return (int)(((int64_t)B * c.top_k + bm - 1) / bm) + c.E;
}

// Lay the MoE workspace for batch B out from `base` (nullptr: sizes only);
// returns the bytes used. Every array starts on a 256-byte boundary.
size_t carve_moe_ws(const tmx_config& C, int64_t B, void* base, MoeWs* ws) {
  const int Pmax = std::max(C.H, C.T);
  int64_t tiles = 0, xh = 0, part = 0, xq = 0;
  for (int sub = 0; sub < 2; ++sub) {
    tiles = std::max<int64_t>(tiles, (int64_t)positions(C, sub) * moe_max_tiles(C, sub, (int)B));
    xh = std::max<int64_t>(xh, (int64_t)positions(C, sub) * B * width(C, sub));
    part = std::max<int64_t>(part, (int64_t)positions(C, sub) * B * C.top_k * width(C, sub));
    if (C.E > 0 && C.dtype == TMX_MXFP8)
      xq = std::max<int64_t>(xq, (int64_t)positions(C, sub) * B * width(C, sub) / 32 * 33);
  }
  const int64_t rk = B * Pmax * C.top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? static_cast<char*>(base) + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  };
  MoeWs w;
  w.xhat = static_cast<uint16_t*>(take(xh * 2));
  w.idx = static_cast<int32_t*>(take(rk * 4));
  w.gate = static_cast<float*>(take(rk * 4));
  w.rows = static_cast<int*>(take(rk * 4));
  w.tiles = static_cast<int4*>(take(tiles * sizeof(int4)));
  w.ntiles = static_cast<int*>(take(Pmax * 4));
  w.counts = static_cast<int*>(take((int64_t)Pmax * C.E * 4));
  w.qhead = static_cast<int*>(take(8 * 4));
  w.hist = static_cast<int*>(take((int64_t)Pmax * ((B + 63) / 64) * C.E * 4));
  w.part = static_cast<uint16_t*>(take(part * 2));
  w.xq8 = xq ? static_cast<uint8_t*>(take(xq)) : nullptr;
  if (ws) *ws = w;
  return off;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool sublayer_ready(tmx_ctx* c, int layer, int sub) {
  for (int k = 0; k < NKINDS; ++k)
    if (kind_applies(c->cfg, sub, k) && !bank(c, layer, sub, k).loaded) return false;
  return true;
}

tmx_status check_ready(tmx_ctx* c) {
  for (int l = 0; l < c->cfg.L; ++l)
    for (int s = 0; s < 2; ++s)
      if (!sublayer_ready(c, l, s))
        return fail(c, TMX_ERR_STATE, "weights of layer %d sub-layer %d are not all loaded", l, s);
  return TMX_OK;
}

// ---- one sub-layer --------------------------------------------------------------
// Row tiling of the per-position MLP. On the Mix map two adjacent positions
// share a tile (BM/2 rows each): their segments of a token are adjacent in
// the block layout, so the tile reads and writes whole 2*D/H-element runs.
void set_row_tiles(MlpArgs& a, int mode, int sub, int W, int P, int B, int dh_bytes) {
  const int bm = mlp_bm(mode, W);
  a.pair = (sub == TMX_MIX && P % 2 == 0 && mlp_pairs_positions(mode, W)) ? 1 : 0;
  const int rows = a.pair ? bm / 2 : bm;
  a.rtiles = (B + rows - 1) / rows;
  // Unpaired Mix tiles: positions 2q and 2q+1 alternate in the tile order,
  // so the workgroups that read the two halves of a run start side by side
  // (runs shorter than a 128-byte line only)
  const int ppx = (P % 8 == 0) ? P / 8 : P;   // positions per tile range of an XCD
  a.ileave = (sub == TMX_MIX && !a.pair && ppx % 2 == 0 && dh_bytes < 128) ? 1 : 0;
}

// RankMixer: part 0 = the token-mixing half (S), 1 = the FFN half from S,
// 2 = the whole block in one kernel, 3 = the experts' gates from S
tmx_status run_rmx(tmx_ctx* c, int layer, int part, const void* x_in, void* x_out, int B, hipStream_t st,
                   float* gates = nullptr) {
  const tmx_config& cfg = c->cfg;
  RmxArgs a{};
  a.B = B; a.T = cfg.T; a.D = cfg.D; a.dh = cfg.D / cfg.H; a.eps = cfg.eps;
  a.E = cfg.E; a.h_e = cfg.expert_hidden;
  a.hidden = cfg.E > 0 ? cfg.E * cfg.expert_hidden : cfg.hidden_rev;
  a.x = static_cast<const uint16_t*>(x_in);
  a.out = static_cast<uint16_t*>(x_out);
  a.gates = gates;
  auto f = [&](int sub, int k) { return static_cast<const float*>(bank(c, layer, sub, k).ptr); };
  auto h = [&](int k) { return static_cast<const uint16_t*>(bank(c, layer, TMX_REVERT, k).ptr); };
  a.g1 = f(TMX_MIX, TMX_W_NORM_GAIN); a.be1 = f(TMX_MIX, TMX_W_NORM_BIAS);
  a.g2 = f(TMX_REVERT, TMX_W_NORM_GAIN); a.be2 = f(TMX_REVERT, TMX_W_NORM_BIAS);
  if (cfg.E > 0) {
    a.w1 = h(TMX_W_EXP_UP); a.w2 = h(TMX_W_EXP_DOWN); a.b1 = h(TMX_W_EXP_BIAS_UP); a.b2 = h(TMX_W_EXP_BIAS_DOWN);
    a.wr = h(TMX_W_ROUTER);
  } else {
    a.w1 = h(TMX_W_UP); a.w2 = h(TMX_W_DOWN); a.b1 = h(TMX_W_BIAS_UP); a.b2 = h(TMX_W_BIAS_DOWN);
  }
  return launch_timed(c, TMX_KERNEL_RMX_BLOCK, st, "RankMixer launch", [&] { return launch_rmx(a, part, st); });
}

tmx_status run_sublayer(tmx_ctx* c, int layer, int sub, const void* x_in, const void* resid, const void* extra,
                        void* x_out, int B, hipStream_t st, const MoeWs& ws) {
  const tmx_config& cfg = c->cfg;
  const int P = positions(cfg, sub), W = width(cfg, sub);
  RowMap map{cfg.T, cfg.D, cfg.D / cfg.H, sub == TMX_MIX ? 1 : 0};
  if (sub == TMX_MIX) resid = x_in;   // H itself, read through the Mix map
  const float* gain = static_cast<const float*>(bank(c, layer, sub, TMX_W_NORM_GAIN).ptr);

  if (cfg.dtype == TMX_F32) {
    F32Args a{};
    a.B = B; a.P = P; a.W = W; a.hidden = is_moe(cfg) ? 0 : dense_hidden(cfg, sub);
    a.E = cfg.E; a.top_k = cfg.top_k; a.expert_hidden = cfg.expert_hidden; a.shared_hidden = cfg.shared_hidden;
    a.alpha = c->alpha; a.eps = cfg.eps; a.map = map;
    a.x = static_cast<const float*>(x_in); a.gain = gain;
    a.resid = static_cast<const float*>(resid); a.extra = static_cast<const float*>(extra);
    a.out = static_cast<float*>(x_out);
    auto w = [&](int k) { return static_cast<const float*>(bank(c, layer, sub, k).ptr); };
    a.w_up = w(TMX_W_UP); a.w_gate = w(TMX_W_GATE); a.w_down = w(TMX_W_DOWN);
    a.w_router = w(TMX_W_ROUTER); a.e_up = w(TMX_W_EXP_UP); a.e_gate = w(TMX_W_EXP_GATE);
    a.e_down = w(TMX_W_EXP_DOWN); a.s_up = w(TMX_W_SH_UP); a.s_gate = w(TMX_W_SH_GATE); a.s_down = w(TMX_W_SH_DOWN);
    return launch_timed(c, TMX_KERNEL_F32, st, "f32 sub-layer launch", [&] { return launch_f32_sublayer(a, st); });
  }

  MlpArgs a{};
  a.B = B; a.P = P; a.map = map; a.eps = cfg.eps;
  a.x = static_cast<const uint16_t*>(x_in); a.gain = gain;
  a.resid = static_cast<const uint16_t*>(resid); a.extra = static_cast<const uint16_t*>(extra);
  a.out = static_cast<uint16_t*>(x_out);
  if (!is_moe(cfg)) {
    a.hidden = dense_hidden(cfg, sub);
    a.wgu = static_cast<const uint16_t*>(storage(c, layer, sub, TMX_W_GATE).ptr);
    a.wd = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_DOWN).ptr);
    set_row_tiles(a, MLP_DENSE, sub, W, P, B, map.dh * 2);
    if (cfg.dtype == TMX_MXFP8) {
      a.wsc = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.wgu) +
                                                (size_t)2 * kind_elems(cfg, sub, TMX_W_GATE));
      a.wrec = mx_rec(cfg, sub, TMX_W_GATE);
      return launch_timed(c, TMX_KERNEL_MLP_DENSE, st, "dense MXFP8 MLP launch", [&] {
        return launch_mlp_mx(MLP_DENSE, W, a, (a.pair ? P / 2 : P) * a.rtiles, c->workers, st);
      });
    }
    return launch_timed(c, TMX_KERNEL_MLP_DENSE, st, "dense MLP launch",
                        [&] { return launch_mlp(MLP_DENSE, W, a, (a.pair ? P / 2 : P) * a.rtiles, c->workers, st); });
  }

  // MoE: norm + route -> bucket -> routed experts -> shared expert + combine
  const int bm = moe_bm(cfg, sub);
  const bool mx = cfg.dtype == TMX_MXFP8;
  const bool wide = mx ? routed_wide_mx_rows(W, cfg.expert_hidden) > 0 : routed_wide_rows(W, cfg.expert_hidden) > 0;
  RouteArgs r{};
  r.B = B; r.P = P; r.E = cfg.E; r.top_k = cfg.top_k; r.alpha = c->alpha; r.eps = cfg.eps; r.map = map;
  r.x = static_cast<const uint16_t*>(x_in); r.gain = gain;
  r.wr = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_ROUTER).ptr);
  r.xhat = ws.xhat; r.idx = ws.idx; r.gate = ws.gate; r.hist = ws.hist;
  if (mx) {   // the expert kernels read x_hat in MXFP8 only
    r.xhat = nullptr;
    r.xq8 = ws.xq8;
    r.xe8 = ws.xq8 + (size_t)P * B * W;
  }
  tmx_status s = launch_timed(c, TMX_KERNEL_ROUTER, st, "router launch", [&] { return launch_norm_route(W, r, st); });
  if (s != TMX_OK) return s;

  BucketArgs k{};
  k.B = B; k.P = P; k.E = cfg.E; k.top_k = cfg.top_k; k.bm = bm; k.max_tiles = moe_max_tiles(cfg, sub, B);
  k.idx = ws.idx; k.rows = ws.rows; k.tiles = ws.tiles; k.ntiles = ws.ntiles; k.counts = ws.counts;
  k.qhead = ws.qhead; k.hist = ws.hist;
  s = launch_timed(c, TMX_KERNEL_BUCKET, st, "bucket launch", [&] { return launch_bucket(k, st); });
  if (s != TMX_OK) return s;

  a.xhat = mx ? nullptr : ws.xhat; a.top_k = cfg.top_k; a.E = cfg.E; a.max_tiles = k.max_tiles;
  a.xq8 = r.xq8; a.xe8 = r.xe8;
  a.rows = ws.rows; a.tiles = ws.tiles; a.ntiles = ws.ntiles; a.gate = ws.gate; a.part = ws.part;
  a.qhead = ws.qhead;
  a.hidden = cfg.expert_hidden;
  a.wgu = static_cast<const uint16_t*>(storage(c, layer, sub, TMX_W_EXP_GATE).ptr);
  a.wd = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_EXP_DOWN).ptr);
  if (mx) {
    a.wsc = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.wgu) +
                                              (size_t)2 * kind_elems(cfg, sub, TMX_W_EXP_GATE));
    a.wrec = mx_rec(cfg, sub, TMX_W_EXP_GATE);
  }
  s = launch_timed(c, TMX_KERNEL_MLP_ROUTED, st, "routed MLP launch", [&] {
    if (mx)
      return wide ? launch_routed_wide_mx(a, P * a.max_tiles, c->workers, st)
                  : launch_mlp_mx(MLP_ROUTED, W, a, P * a.max_tiles, c->workers, st);
    return wide ? launch_routed_wide(a, P * a.max_tiles, c->workers, st)
                : launch_mlp(MLP_ROUTED, W, a, P * a.max_tiles, c->workers, st);
  });
  if (s != TMX_OK) return s;

  a.hidden = cfg.shared_hidden;
  a.wgu = static_cast<const uint16_t*>(storage(c, layer, sub, TMX_W_SH_GATE).ptr);
  a.wd = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_SH_DOWN).ptr);
  if (mx) {
    a.wsc = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.wgu) +
                                              (size_t)2 * kind_elems(cfg, sub, TMX_W_SH_GATE));
    a.wrec = mx_rec(cfg, sub, TMX_W_SH_GATE);
  }
  set_row_tiles(a, MLP_SHARED, sub, W, P, B, map.dh * 2);
  // The shared-expert tiles are all alike, so a persistent launch keeps its
  // workgroups in step: every combine epilogue (k expert rows + residual per
  // row, HBM-bound) would run at once while no MFMA runs. With 4 or more
  // tiles per workgroup, every other workgroup of an XCD starts about one
  // main loop (1.3 x the tile's MFMA clocks) late, so half of them combine
  // while the other half compute.
  const int sh_tiles = (a.pair ? P / 2 : P) * a.rtiles;
  const int sh_grid = std::max(1, std::min(sh_tiles, c->workers & ~7));
  // (MXFP8 MFMAs take half the clocks per multiply-add)
  const double mfma_clk = (double)mlp_bm(MLP_SHARED, W) * W * 3.0 * cfg.shared_hidden / (16384.0 * 4.0) * 32.0 /
                          (mx ? 2.0 : 1.0);
  a.stagger = sh_tiles >= 4 * sh_grid ? (int)(1.3 * mfma_clk) : 0;
  return launch_timed(c, TMX_KERNEL_MLP_SHARED, st, "shared MLP launch", [&] {
    return mx ? launch_mlp_mx(MLP_SHARED, W, a, sh_tiles, c->workers, st)
              : launch_mlp(MLP_SHARED, W, a, sh_tiles, c->workers, st);
  });
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tmx_status check_act(tmx_ctx* c, const void* p, const char* name) {
  if (!p) return fail(c, TMX_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(c, TMX_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return TMX_OK;
}

tmx_status check_B(tmx_ctx* c, int B) {
  if (B < 1 || B > c->cfg.B_max)
    return fail(c, TMX_ERR_INVALID_ARG, "B = %d outside [1, B_max = %d]", B, c->cfg.B_max);
  return TMX_OK;
}

bool overlaps(const void* a, const void* b, size_t n) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + n && y < x + n;
}

}  // namespace

// =============================================================================
// C ABI
// =============================================================================

extern "C" {

const char* tmx_last_error(const tmx_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

tmx_status tmx_create(const tmx_config* cfg, int device, tmx_ctx** out) {
  if (!out) return fail(nullptr, TMX_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  tmx_status s = validate_config(cfg);
  if (s != TMX_OK) return s;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev == 0) {
    (void)hipGetLastError();
    return fail(nullptr, TMX_ERR_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  }
  if (device < 0 || device >= ndev)
    return fail(nullptr, TMX_ERR_INVALID_ARG, "device %d outside [0, %d)", device, ndev);
  if ((e = hipSetDevice(device)) != hipSuccess)
    return fail(nullptr, TMX_ERR_DEVICE, "hipSetDevice(%d): %s", device, hipGetErrorString(e));

  tmx_ctx* c = new tmx_ctx();
  c->cfg = *cfg;
  c->device = device;
  if ((e = hipDeviceGetAttribute(&c->workers, hipDeviceAttributeMultiprocessorCount, device)) != hipSuccess) {
    delete c;
    return fail(nullptr, TMX_ERR_DEVICE, "compute-unit count: %s", hipGetErrorString(e));
  }
  setup_scratch(device);
  c->alpha = cfg->E > 0 ? (cfg->alpha != 0.f ? cfg->alpha : (float)cfg->E / (float)cfg->top_k) : 0.f;
  c->banks.resize((size_t)cfg->L * 2 * NKINDS);
  const tmx_config& C = c->cfg;
  const size_t es = esize(C);

  auto bail = [&](tmx_status st) {
    g_create_error = c->err;
    release(c);
    delete c;
    return st;
  };

  for (int l = 0; l < C.L; ++l)
    for (int sub = 0; sub < 2; ++sub)
      for (int k = 0; k < NKINDS; ++k) {
        if (!kind_applies(C, sub, k)) continue;
        Bank& b = bank(c, l, sub, k);
        b.elems = kind_elems(C, sub, k);
        if (is_norm(k)) {
          s = dev_alloc(c, &b.ptr, b.elems * sizeof(float), "norm parameters");
          if (s != TMX_OK) return bail(s);
          std::vector<float> init(b.elems, k == TMX_W_NORM_GAIN ? 1.0f : 0.0f);
          if ((e = hipMemcpy(b.ptr, init.data(), b.elems * sizeof(float), hipMemcpyHostToDevice)) != hipSuccess)
            return bail(fail(c, TMX_ERR_DEVICE, "norm init: %s", hipGetErrorString(e)));
          b.loaded = true;
          continue;
        }
        if (is_bias(k)) {
          // the experts' second biases are stored packed and stacked twice
          const size_t n = k == TMX_W_EXP_BIAS_DOWN ? 2 * b.elems : b.elems;
          s = dev_alloc(c, &b.ptr, n * es, "biases");
          if (s != TMX_OK) return bail(s);
          std::vector<uint16_t> zero(n, 0);   // bf16 +0 (also as packed fragments)
          if ((e = hipMemcpy(b.ptr, zero.data(), n * es, hipMemcpyHostToDevice)) != hipSuccess)
            return bail(fail(c, TMX_ERR_DEVICE, "bias init: %s", hipGetErrorString(e)));
          b.loaded = true;
          continue;
        }
        if (is_rmx(C)) {   // W1 / W2 (router, experts' W1 / W2), one fragment buffer each
          if ((s = dev_alloc(c, &b.ptr, b.elems * es, "weights")) != TMX_OK) return bail(s);
          continue;
        }
        if (C.dtype != TMX_F32 && (k == TMX_W_UP || k == TMX_W_EXP_UP || k == TMX_W_SH_UP)) continue;
        size_t n = b.elems;
        if (C.dtype != TMX_F32 && (k == TMX_W_GATE || k == TMX_W_EXP_GATE || k == TMX_W_SH_GATE)) n *= 2;
        size_t bytes = n * es;
        // MXFP8: one byte per weight; the gate bank also holds the scale
        // records of its family's gate, up and down matrices (the router
        // stays bf16)
        if (C.dtype == TMX_MXFP8 && mx_gate_kind(k) >= 0)
          bytes = n + (mx_gate_kind(k) == k ? mx_rec_bytes(C, sub, k) : 0);
        s = dev_alloc(c, &b.ptr, bytes, "weights");
        if (s != TMX_OK) return bail(s);
      }

  const int64_t act = (int64_t)C.B_max * C.T * C.D;
  for (int i = 0; i < 3; ++i)
    if ((s = dev_alloc(c, &c->act[i], act * es, "activations")) != TMX_OK) return bail(s);
  if ((s = dev_alloc(c, &c->xrev, act * es, "activations")) != TMX_OK) return bail(s);

  if (C.E > 0 && (C.dtype == TMX_BF16 || C.dtype == TMX_MXFP8)) {
    void* base = nullptr;
    if ((s = dev_alloc(c, &base, carve_moe_ws(C, C.B_max, nullptr, nullptr), "MoE workspace")) != TMX_OK)
      return bail(s);
    carve_moe_ws(C, C.B_max, base, &c->ws);
  }
  *out = c;
  return TMX_OK;
}

tmx_status tmx_destroy(tmx_ctx* ctx) {
  if (!ctx) return TMX_OK;
  (void)hipSetDevice(ctx->device);
  for (auto& t : ctx->pending) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.end);
  }
  for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
  release(ctx);
  delete ctx;
  return TMX_OK;
}

tmx_status tmx_load_weights(tmx_ctx* c, int layer, int sub, int kind, const void* src, size_t nbytes,
                            void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  const tmx_config& C = c->cfg;
  if (layer < 0 || layer >= C.L) return fail(c, TMX_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, C.L);
  if (sub != TMX_MIX && sub != TMX_REVERT) return fail(c, TMX_ERR_INVALID_ARG, "sublayer must be 0 or 1, got %d", sub);
  if (kind < 0 || kind >= NKINDS) return fail(c, TMX_ERR_INVALID_ARG, "unknown weight kind %d", kind);
  if (!kind_applies(C, sub, kind))
    return fail(c, TMX_ERR_INVALID_ARG, "weight kind %d does not apply to sub-layer %d of a %s context", kind, sub,
                is_rmx(C) ? "RankMixer" : is_moe(C) ? "MoE" : "dense");
  if (!src) return fail(c, TMX_ERR_INVALID_ARG, "src is NULL");
  const size_t es = esize(C);
  const size_t elems = kind_elems(C, sub, kind);
  if (nbytes != elems * es)
    return fail(c, TMX_ERR_INVALID_ARG, "nbytes %zu != expected %zu for kind %d", nbytes, elems * es, kind);

  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(e));
  hipStream_t st = as_stream(stream);

  bool src_dev = false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, src) == hipSuccess)
    src_dev = attr.type == hipMemoryTypeDevice;
  (void)hipGetLastError();

  Bank& b = bank(c, layer, sub, kind);
  if (is_norm(kind)) {
    std::vector<float> g(elems);
    std::vector<unsigned char> raw(nbytes);
    e = hipMemcpy(raw.data(), src, nbytes, src_dev ? hipMemcpyDeviceToHost : hipMemcpyHostToHost);
    if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "gain copy: %s", hipGetErrorString(e));
    for (size_t i = 0; i < elems; ++i) {
      if (es == 4) {
        memcpy(&g[i], &raw[i * 4], 4);
      } else {
        uint16_t h;
        memcpy(&h, &raw[i * 2], 2);
        uint32_t u = (uint32_t)h << 16;
        memcpy(&g[i], &u, 4);
      }
    }
    e = hipMemcpy(b.ptr, g.data(), elems * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "gain upload: %s", hipGetErrorString(e));
    b.loaded = true;
    return TMX_OK;
  }

  if (C.dtype == TMX_F32 || kind == TMX_W_BIAS_UP || kind == TMX_W_BIAS_DOWN || kind == TMX_W_EXP_BIAS_UP) {
    e = hipMemcpyAsync(b.ptr, src, nbytes, src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "weight copy: %s", hipGetErrorString(e));
    b.loaded = true;
    return TMX_OK;
  }

  // bf16: stage on the device, then repack into MFMA fragments (the experts'
  // second biases staged twice per token: [T][2E][D])
  const bool twice = kind == TMX_W_EXP_BIAS_DOWN;
  void* stage = nullptr;
  e = hipMalloc(&stage, twice ? 2 * nbytes : nbytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, e == hipErrorOutOfMemory ? TMX_ERR_OOM : TMX_ERR_DEVICE, "staging buffer: %s",
                hipGetErrorString(e));
  }
  int64_t G = 0;
  int K = 0, N = 0;
  if (twice) {
    const size_t row = (size_t)C.E * C.D * es;   // one token's [E][D]
    for (int half = 0; half < 2 && e == hipSuccess; ++half)
      e = hipMemcpy2DAsync(static_cast<char*>(stage) + half * row, 2 * row, src, row, row, C.T,
                           src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, st);
    G = C.T; K = 2 * C.E; N = C.D;
  } else {
    e = hipMemcpyAsync(stage, src, nbytes, src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, st);
    bank_dims(C, sub, kind, &G, &K, &N);
  }
  const bool gu = kind == TMX_W_UP || kind == TMX_W_GATE || kind == TMX_W_EXP_UP || kind == TMX_W_EXP_GATE ||
                  kind == TMX_W_SH_UP || kind == TMX_W_SH_GATE;
  const int which = (kind == TMX_W_UP || kind == TMX_W_EXP_UP || kind == TMX_W_SH_UP) ? 1 : 0;
  if (e == hipSuccess && C.dtype == TMX_MXFP8 && mx_gate_kind(kind) >= 0) {
    const int gk = mx_gate_kind(kind);
    uint8_t* gub = static_cast<uint8_t*>(bank(c, layer, sub, gk).ptr);
    uint8_t* rec = gub + (size_t)2 * kind_elems(C, sub, gk);
    const bool down = !gu;
    uint8_t* dst = down ? static_cast<uint8_t*>(bank(c, layer, sub, kind).ptr) : gub;
    e = launch_pack_mx(static_cast<const uint16_t*>(stage), dst, rec, (int)G, K, N, down ? 1 : 0, which,
                       mx_rec(C, sub, gk), st);
  } else if (e == hipSuccess && is_rmx(C))
    e = launch_pack(static_cast<const uint16_t*>(stage), static_cast<uint16_t*>(b.ptr), (int)G, K, N,
                    kind == TMX_W_ROUTER ? 1 : 2, 0, kind == TMX_W_ROUTER ? FRAG_16x16x32 : FRAG_32x32x16, st);
  else if (e == hipSuccess)
    e = launch_pack(static_cast<const uint16_t*>(stage), static_cast<uint16_t*>(storage(c, layer, sub, kind).ptr),
                    (int)G, K, N, gu ? 0 : 1, which, kind == TMX_W_ROUTER ? FRAG_16x16x32 : FRAG_32x32x16, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  (void)hipFree(stage);
  if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "weight upload/pack: %s", hipGetErrorString(e));
  b.loaded = true;
  return TMX_OK;
}

}  // extern "C"

namespace {

tmx_status check_sublayer_args(tmx_ctx* c, int layer, int sub, const void* x_in, const void* resid,
                               const void* extra, void* x_out, int B) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if (layer < 0 || layer >= c->cfg.L) return fail(c, TMX_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c->cfg.L);
  if (sub != TMX_MIX && sub != TMX_REVERT) return fail(c, TMX_ERR_INVALID_ARG, "sublayer must be 0 or 1");
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, x_in, "x_in")) != TMX_OK) return s;
  if ((s = check_act(c, x_out, "x_out")) != TMX_OK) return s;
  const size_t bytes = (size_t)B * c->cfg.T * c->cfg.D * esize(c->cfg);
  if (sub == TMX_MIX || is_rmx(c->cfg)) {
    if (resid || extra) return fail(c, TMX_ERR_INVALID_ARG, "this sub-layer takes no resid/extra (pass NULL)");
  } else {
    if ((s = check_act(c, resid, "resid")) != TMX_OK) return s;
    if (extra && !aligned16(extra)) return fail(c, TMX_ERR_INVALID_ARG, "extra must be 16-byte aligned");
    if (overlaps(resid, x_out, bytes) || (extra && overlaps(extra, x_out, bytes)))
      return fail(c, TMX_ERR_INVALID_ARG, "x_out overlaps an input");
  }
  if (overlaps(x_in, x_out, bytes)) return fail(c, TMX_ERR_INVALID_ARG, "x_in and x_out overlap");
  if (!sublayer_ready(c, layer, sub))
    return fail(c, TMX_ERR_STATE, "weights of layer %d sub-layer %d are not all loaded", layer, sub);
  return TMX_OK;
}

}  // namespace

extern "C" {

tmx_status tmx_sublayer_forward(tmx_ctx* c, int layer, int sub, const void* x_in, const void* resid,
                                const void* extra, void* x_out, int B, void* stream) {
  tmx_status s = check_sublayer_args(c, layer, sub, x_in, resid, extra, x_out, B);
  if (s != TMX_OK) return s;
  (void)hipSetDevice(c->device);
  if (is_rmx(c->cfg)) return run_rmx(c, layer, sub, x_in, x_out, B, as_stream(stream));
  return run_sublayer(c, layer, sub, x_in, resid, extra, x_out, B, as_stream(stream), c->ws);
}

tmx_status tmx_sublayer_forward_noalloc(tmx_ctx* c, int layer, int sub, const void* x_in, const void* resid,
                                        const void* extra, void* x_out, int B, void* stream) {
  tmx_status s = check_sublayer_args(c, layer, sub, x_in, resid, extra, x_out, B);
  if (s != TMX_OK) return s;
  const tmx_config& C = c->cfg;
  MoeWs ws;
  if (is_moe(C) && !is_rmx(C) && (C.dtype == TMX_BF16 || C.dtype == TMX_MXFP8)) {
    const size_t need = carve_moe_ws(C, B, nullptr, nullptr);
    if (need > TMX_SCRATCH_BYTES) {
      int bmax = 0;
      for (int lo = 1, hi = C.B_max; lo <= hi;) {   // largest B whose workspace fits
        const int mid = lo + (hi - lo) / 2;
        if (carve_moe_ws(C, mid, nullptr, nullptr) <= TMX_SCRATCH_BYTES) {
          bmax = mid;
          lo = mid + 1;
        } else {
          hi = mid - 1;
        }
      }
      return fail(c, TMX_ERR_INVALID_ARG,
                  "B = %d needs %zu bytes of MoE workspace; the static scratch holds %zu (B <= %d for this context)",
                  B, need, TMX_SCRATCH_BYTES, bmax);
    }
    void* base = (c->device >= 0 && c->device < TMX_SCRATCH_DEVICES) ? g_scratch_ptr[c->device] : nullptr;
    if (!base)
      return fail(c, TMX_ERR_DEVICE, "static scratch of device %d unavailable: %s", c->device,
                  hipGetErrorString(c->device >= 0 && c->device < TMX_SCRATCH_DEVICES ? g_scratch_err[c->device]
                                                                                     : hipErrorInvalidDevice));
    carve_moe_ws(C, B, base, &ws);
  }
  (void)hipSetDevice(c->device);
  if (is_rmx(C)) return run_rmx(c, layer, sub, x_in, x_out, B, as_stream(stream));
  return run_sublayer(c, layer, sub, x_in, resid, extra, x_out, B, as_stream(stream), ws);
}

tmx_status tmx_block_stack_forward(tmx_ctx* c, const void* x_in, void* x_out, int B, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, x_in, "x_in")) != TMX_OK) return s;
  if ((s = check_act(c, x_out, "x_out")) != TMX_OK) return s;
  const size_t bytes = (size_t)B * c->cfg.T * c->cfg.D * esize(c->cfg);
  if (overlaps(x_in, x_out, bytes)) return fail(c, TMX_ERR_INVALID_ARG, "x_in and x_out overlap");
  if ((s = check_ready(c)) != TMX_OK) return s;
  (void)hipSetDevice(c->device);
  hipStream_t st = as_stream(stream);
  const int L = c->cfg.L, g = c->cfg.inter_residual_gap;
  if (is_rmx(c->cfg)) {
    const void* cur = x_in;
    for (int l = 1; l <= L; ++l) {
      void* dst = l == L ? x_out : c->act[l & 1];
      if ((s = run_rmx(c, l - 1, 2, cur, dst, B, st)) != TMX_OK) return s;
      cur = dst;
    }
    return TMX_OK;
  }
  const void* cur = x_in;    // Y_{l-1}
  const void* save = x_in;   // Y_{l-g}: the output of the last multiple of g
  for (int l = 1; l <= L; ++l) {
    if ((s = run_sublayer(c, l - 1, TMX_MIX, cur, nullptr, nullptr, c->xrev, B, st, c->ws)) != TMX_OK) return s;
    const bool inter = g > 0 && l % g == 0 && l < L;
    void* dst = x_out;
    if (l < L)
      for (void* cand : c->act)
        if (cand != cur && cand != save) {
          dst = cand;
          break;
        }
    if ((s = run_sublayer(c, l - 1, TMX_REVERT, c->xrev, cur, inter ? save : nullptr, dst, B, st, c->ws)) != TMX_OK)
      return s;
    if (g > 0 && l % g == 0) save = dst;
    cur = dst;
  }
  return TMX_OK;
}

tmx_status tmx_moe_route(tmx_ctx* c, int layer, int sub, const void* x, int B, int32_t* idx, float* gate,
                         void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  const tmx_config& C = c->cfg;
  if (!is_moe(C) || is_rmx(C))
    return fail(c, TMX_ERR_UNSUPPORTED, "tmx_moe_route needs a TokenMixer-Large MoE context (top-k softmax router)");
  tmx_status s;
  if (layer < 0 || layer >= C.L) return fail(c, TMX_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, C.L);
  if (sub != TMX_MIX && sub != TMX_REVERT) return fail(c, TMX_ERR_INVALID_ARG, "sublayer must be 0 or 1");
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, x, "x")) != TMX_OK) return s;
  if (!idx || !gate) return fail(c, TMX_ERR_INVALID_ARG, "idx and gate must be non-NULL");
  if (!bank(c, layer, sub, TMX_W_ROUTER).loaded)
    return fail(c, TMX_ERR_STATE, "router of layer %d sub-layer %d is not loaded", layer, sub);
  (void)hipSetDevice(c->device);
  hipStream_t st = as_stream(stream);
  const int P = positions(C, sub), W = width(C, sub);
  RowMap map{C.T, C.D, C.D / C.H, sub == TMX_MIX ? 1 : 0};
  const float* gain = static_cast<const float*>(bank(c, layer, sub, TMX_W_NORM_GAIN).ptr);
  if (C.dtype == TMX_F32) {
    F32Args a{};
    a.B = B; a.P = P; a.W = W; a.E = C.E; a.top_k = C.top_k; a.expert_hidden = C.expert_hidden;
    a.shared_hidden = C.shared_hidden; a.alpha = c->alpha; a.eps = C.eps; a.map = map;
    a.x = static_cast<const float*>(x); a.gain = gain;
    a.w_router = static_cast<const float*>(bank(c, layer, sub, TMX_W_ROUTER).ptr);
    a.idx = idx; a.gate_out = gate; a.route_only = 1;
    return check_launch(c, launch_f32_sublayer(a, st), "f32 router launch");
  }
  RouteArgs r{};
  r.B = B; r.P = P; r.E = C.E; r.top_k = C.top_k; r.alpha = c->alpha; r.eps = C.eps; r.map = map;
  r.x = static_cast<const uint16_t*>(x); r.gain = gain;
  r.wr = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_ROUTER).ptr);
  r.xhat = nullptr; r.idx = idx; r.gate = gate;
  return check_launch(c, launch_norm_route(W, r, st), "router launch");
}

tmx_status tmx_moe_buckets(tmx_ctx* c, int layer, int sub, const void* x, int B, void* xhat, int32_t* counts,
                           int32_t* rows, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  const tmx_config& C = c->cfg;
  if (!is_moe(C) || is_rmx(C) || (C.dtype != TMX_BF16 && C.dtype != TMX_MXFP8))
    return fail(c, TMX_ERR_UNSUPPORTED, "tmx_moe_buckets needs a bf16 or MXFP8 TokenMixer-Large MoE context");
  tmx_status s;
  if (layer < 0 || layer >= C.L) return fail(c, TMX_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, C.L);
  if (sub != TMX_MIX && sub != TMX_REVERT) return fail(c, TMX_ERR_INVALID_ARG, "sublayer must be 0 or 1");
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, x, "x")) != TMX_OK) return s;
  if (xhat && !aligned16(xhat)) return fail(c, TMX_ERR_INVALID_ARG, "xhat must be 16-byte aligned");
  if (!bank(c, layer, sub, TMX_W_ROUTER).loaded)
    return fail(c, TMX_ERR_STATE, "router of layer %d sub-layer %d is not loaded", layer, sub);
  (void)hipSetDevice(c->device);
  hipStream_t st = as_stream(stream);
  const int P = positions(C, sub), W = width(C, sub);
  RouteArgs r{};
  r.B = B; r.P = P; r.E = C.E; r.top_k = C.top_k; r.alpha = c->alpha; r.eps = C.eps;
  r.map = RowMap{C.T, C.D, C.D / C.H, sub == TMX_MIX ? 1 : 0};
  r.x = static_cast<const uint16_t*>(x);
  r.gain = static_cast<const float*>(bank(c, layer, sub, TMX_W_NORM_GAIN).ptr);
  r.wr = static_cast<const uint16_t*>(bank(c, layer, sub, TMX_W_ROUTER).ptr);
  r.xhat = c->ws.xhat; r.idx = c->ws.idx; r.gate = c->ws.gate; r.hist = c->ws.hist;
  if ((s = check_launch(c, launch_norm_route(W, r, st), "router launch")) != TMX_OK) return s;
  BucketArgs k{};
  k.B = B; k.P = P; k.E = C.E; k.top_k = C.top_k; k.bm = moe_bm(C, sub); k.max_tiles = moe_max_tiles(C, sub, B);
  k.idx = c->ws.idx; k.rows = c->ws.rows; k.tiles = c->ws.tiles; k.ntiles = c->ws.ntiles; k.counts = c->ws.counts;
  k.qhead = c->ws.qhead; k.hist = c->ws.hist;
  if ((s = check_launch(c, launch_bucket(k, st), "bucket launch")) != TMX_OK) return s;
  hipError_t e = hipSuccess;
  if (xhat) e = hipMemcpyAsync(xhat, c->ws.xhat, (size_t)P * B * W * 2, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && counts)
    e = hipMemcpyAsync(counts, c->ws.counts, (size_t)P * C.E * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && rows)
    e = hipMemcpyAsync(rows, c->ws.rows, (size_t)P * B * C.top_k * 4, hipMemcpyDeviceToDevice, st);
  return check_launch(c, e, "workspace copy");
}

tmx_status tmx_relu_route(tmx_ctx* c, int layer, const void* s, int B, float* gates, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  const tmx_config& C = c->cfg;
  if (!is_rmx(C) || !is_moe(C))
    return fail(c, TMX_ERR_UNSUPPORTED, "tmx_relu_route needs a RankMixer context with ReLU-routed experts");
  tmx_status st;
  if (layer < 0 || layer >= C.L) return fail(c, TMX_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, C.L);
  if ((st = check_B(c, B)) != TMX_OK) return st;
  if ((st = check_act(c, s, "s")) != TMX_OK) return st;
  if (!gates) return fail(c, TMX_ERR_INVALID_ARG, "gates is NULL");
  if (!bank(c, layer, TMX_REVERT, TMX_W_ROUTER).loaded)
    return fail(c, TMX_ERR_STATE, "router of layer %d is not loaded", layer);
  (void)hipSetDevice(c->device);
  return run_rmx(c, layer, 3, s, nullptr, B, as_stream(stream), gates);
}

tmx_status tmx_debug_permute(tmx_ctx* c, const void* in, void* out, int B, int inverse, int form, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if (!in || !out) return fail(c, TMX_ERR_INVALID_ARG, "in/out must be non-NULL");
  if (inverse != 0 && inverse != 1) return fail(c, TMX_ERR_INVALID_ARG, "inverse must be 0 or 1");
  if (form < TMX_PERM_ELEMENT || form > TMX_PERM_CURSOR)
    return fail(c, TMX_ERR_INVALID_ARG, "form must be 0, 1 or 2, got %d", form);
  const tmx_config& C = c->cfg;
  if (form != TMX_PERM_ELEMENT) {
    if (!aligned16(in) || !aligned16(out)) return fail(c, TMX_ERR_INVALID_ARG, "in/out must be 16-byte aligned");
    if ((C.D / C.H) % 8 != 0 || (C.T * (C.D / C.H)) % 32 != 0)
      return fail(c, TMX_ERR_UNSUPPORTED, "8-column unit forms need D/H %% 8 == 0 and T*D/H %% 32 == 0");
  }
  const size_t bytes = (size_t)B * C.T * C.D * esize(C);
  if (overlaps(in, out, bytes)) return fail(c, TMX_ERR_INVALID_ARG, "in and out overlap");
  (void)hipSetDevice(c->device);
  return check_launch(c, launch_permute(in, out, B, C.T, C.D, C.H, (int)esize(C), inverse, form, as_stream(stream)),
                      "permute launch");
}

tmx_status tmx_set_model_io(tmx_ctx* c, const int32_t* group_widths, int n_groups, int tok_hidden,
                            int head_hidden) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  const tmx_config& C = c->cfg;
  if (c->io.set) return fail(c, TMX_ERR_STATE, "the model's tokenizer and head are already set");
  if (!group_widths) return fail(c, TMX_ERR_INVALID_ARG, "group_widths is NULL");
  if (n_groups != C.T - 1 || n_groups < 1)
    return fail(c, TMX_ERR_INVALID_ARG, "need T - 1 = %d semantic groups (token 0 is the global token), got %d",
                C.T - 1, n_groups);
  int64_t F = 0;
  for (int i = 0; i < n_groups; ++i) {
    if (group_widths[i] < 1) return fail(c, TMX_ERR_INVALID_ARG, "group %d has width %d", i, group_widths[i]);
    F += group_widths[i];
  }
  if (tok_hidden < 1 || head_hidden < 1) return fail(c, TMX_ERR_INVALID_ARG, "hidden widths must be >= 1");
  if (F > (1 << 20)) return fail(c, TMX_ERR_INVALID_ARG, "embedding width %lld too large", (long long)F);
  if (C.dtype != TMX_BF16 && C.dtype != TMX_MXFP8)
    return fail(c, TMX_ERR_UNSUPPORTED, "the tokenizer and head run on bf16 activations");
  for (int i = 0; i < n_groups; ++i)
    if (group_widths[i] % 32 != 0)
      return fail(c, TMX_ERR_UNSUPPORTED, "group widths must be multiples of 32 (group %d: %d)", i, group_widths[i]);
  if (!io_width_supported(C.D) || !io_tok_hidden_supported(tok_hidden) || !io_head_hidden_supported(head_hidden))
    return fail(c, TMX_ERR_UNSUPPORTED,
                "tokenizer/head need D in {128, 256, 512, 768}, tok_hidden in {128, 256, 512, 768} and head_hidden "
                "in {128, 256, 512} (got %d, %d, %d)", C.D, tok_hidden, head_hidden);
  (void)hipSetDevice(c->device);
  {
    auto& io = c->io;
    const int T = C.T;
    std::vector<int4> pos(T);
    int64_t frag = 0, off = 0;
    for (int t = 0; t < T; ++t) {
      const int K = t == 0 ? (int)F : group_widths[t - 1];
      pos[t] = make_int4(t == 0 ? 0 : (int)off, K, (int)frag, 0);
      if (t > 0) off += K;
      frag += (int64_t)(K / 16) * (tok_hidden / 32);
    }
    tmx_status s;
    const int64_t act = (int64_t)C.B_max * C.T * C.D * 2;
    if ((s = dev_alloc(c, (void**)&io.pos, T * sizeof(int4), "tokenizer table")) != TMX_OK ||
        (s = dev_alloc(c, (void**)&io.w1, frag * FRAG_ELEMS * 2, "tokenizer W1")) != TMX_OK ||
        (s = dev_alloc(c, (void**)&io.w2, (size_t)T * tok_hidden * C.D * 2, "tokenizer W2")) != TMX_OK ||
        (s = dev_alloc(c, (void**)&io.hw1, (size_t)C.D * head_hidden * 2, "head W1")) != TMX_OK ||
        (s = dev_alloc(c, (void**)&io.hw2, (size_t)head_hidden * 2, "head w2")) != TMX_OK ||
        (s = dev_alloc(c, &io.xbuf, act, "model tokens")) != TMX_OK ||
        (s = dev_alloc(c, &io.ybuf, act, "model stack output")) != TMX_OK)
      return s;
    hipError_t e = hipMemcpy(io.pos, pos.data(), T * sizeof(int4), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "tokenizer table: %s", hipGetErrorString(e));
    io.widths.assign(group_widths, group_widths + n_groups);
    io.F = (int)F;
    io.h = tok_hidden;
    io.hh = head_hidden;
    io.set = true;
  }
  return TMX_OK;
}

tmx_status tmx_load_io_weights(tmx_ctx* c, int kind, const void* src, size_t nbytes, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  auto& io = c->io;
  const tmx_config& C = c->cfg;
  if (!io.set) return fail(c, TMX_ERR_STATE, "tmx_set_model_io has not been called");
  if (kind < TMX_W_TOK_UP || kind > TMX_W_HEAD_DOWN)
    return fail(c, TMX_ERR_INVALID_ARG, "kind %d is not a tokenizer or head bank", kind);
  if (!src) return fail(c, TMX_ERR_INVALID_ARG, "src is NULL");
  const size_t elems = kind == TMX_W_TOK_UP     ? (size_t)2 * io.F * io.h
                       : kind == TMX_W_TOK_DOWN ? (size_t)C.T * io.h * C.D
                       : kind == TMX_W_HEAD_UP  ? (size_t)C.D * io.hh
                                                : (size_t)io.hh;
  if (nbytes != elems * 2) return fail(c, TMX_ERR_INVALID_ARG, "nbytes %zu != expected %zu", nbytes, elems * 2);
  (void)hipSetDevice(c->device);
  hipStream_t st = as_stream(stream);
  bool src_dev = false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, src) == hipSuccess) src_dev = attr.type == hipMemoryTypeDevice;
  (void)hipGetLastError();
  const hipMemcpyKind mk = src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  hipError_t e;
  if (kind == TMX_W_HEAD_DOWN) {
    e = hipMemcpyAsync(io.hw2, src, nbytes, mk, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  } else {
    void* stage = nullptr;
    e = hipMalloc(&stage, nbytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(c, e == hipErrorOutOfMemory ? TMX_ERR_OOM : TMX_ERR_DEVICE, "staging buffer: %s",
                  hipGetErrorString(e));
    }
    e = hipMemcpyAsync(stage, src, nbytes, mk, st);
    const uint16_t* sp = static_cast<const uint16_t*>(stage);
    if (kind == TMX_W_TOK_UP) {
      // position 0 (global token): rows [0, F); group t: the next d_t rows
      int64_t row = 0, frag = 0;
      for (int t = 0; t < C.T && e == hipSuccess; ++t) {
        const int K = t == 0 ? io.F : io.widths[t - 1];
        e = launch_pack(sp + row * io.h, io.w1 + frag * FRAG_ELEMS, 1, K, io.h, 2, 0, FRAG_32x32x16, st);
        row += K;
        frag += (int64_t)(K / 16) * (io.h / 32);
      }
    } else if (kind == TMX_W_TOK_DOWN) {
      if (e == hipSuccess) e = launch_pack(sp, io.w2, C.T, io.h, C.D, 2, 0, FRAG_32x32x16, st);
    } else {
      if (e == hipSuccess) e = launch_pack(sp, io.hw1, 1, C.D, io.hh, 2, 0, FRAG_32x32x16, st);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipFree(stage);
  }
  if (e != hipSuccess) return fail(c, TMX_ERR_DEVICE, "tokenizer/head upload: %s", hipGetErrorString(e));
  io.loaded[kind - TMX_W_TOK_UP] = true;
  return TMX_OK;
}

}  // extern "C"

namespace {

IoArgs io_args(tmx_ctx* c, int B) {
  IoArgs a{};
  a.B = B; a.T = c->cfg.T; a.D = c->cfg.D; a.F = c->io.F; a.tok_hidden = c->io.h; a.head_hidden = c->io.hh;
  a.tok_pos = c->io.pos; a.tok_w1 = c->io.w1; a.tok_w2 = c->io.w2; a.head_w1 = c->io.hw1; a.head_w2 = c->io.hw2;
  return a;
}

tmx_status check_io(tmx_ctx* c, bool tok, bool head) {
  if (!c->io.set) return fail(c, TMX_ERR_STATE, "tmx_set_model_io has not been called");
  if (tok && !(c->io.loaded[0] && c->io.loaded[1]))
    return fail(c, TMX_ERR_STATE, "the tokenizer weights (TMX_W_TOK_UP, TMX_W_TOK_DOWN) are not loaded");
  if (head && !(c->io.loaded[2] && c->io.loaded[3]))
    return fail(c, TMX_ERR_STATE, "the head weights (TMX_W_HEAD_UP, TMX_W_HEAD_DOWN) are not loaded");
  return TMX_OK;
}

tmx_status run_tokenize(tmx_ctx* c, const void* emb, void* x_out, int B, hipStream_t st) {
  IoArgs a = io_args(c, B);
  a.emb = static_cast<const uint16_t*>(emb);
  a.x_out = static_cast<uint16_t*>(x_out);
  return launch_timed(c, TMX_KERNEL_TOKENIZE, st, "tokenizer launch", [&] { return launch_tokenize(a, st); });
}

tmx_status run_head(tmx_ctx* c, const void* y, float* logits, int B, hipStream_t st) {
  IoArgs a = io_args(c, B);
  a.y = static_cast<const uint16_t*>(y);
  a.logits = logits;
  return launch_timed(c, TMX_KERNEL_HEAD, st, "head launch", [&] { return launch_head(a, st); });
}

}  // namespace

extern "C" {

tmx_status tmx_tokenize(tmx_ctx* c, const void* emb, void* x_out, int B, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, emb, "emb")) != TMX_OK) return s;
  if ((s = check_act(c, x_out, "x_out")) != TMX_OK) return s;
  if ((s = check_io(c, true, false)) != TMX_OK) return s;
  {
    const char* e0 = static_cast<const char*>(emb);
    const char* x0 = static_cast<const char*>(x_out);
    const size_t eb = (size_t)B * c->io.F * 2, xb = (size_t)B * c->cfg.T * c->cfg.D * 2;
    if (e0 < x0 + xb && x0 < e0 + eb) return fail(c, TMX_ERR_INVALID_ARG, "emb and x_out overlap");
  }
  (void)hipSetDevice(c->device);
  return run_tokenize(c, emb, x_out, B, as_stream(stream));
}

tmx_status tmx_head(tmx_ctx* c, const void* y, float* logits, int B, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, y, "y")) != TMX_OK) return s;
  if (!logits) return fail(c, TMX_ERR_INVALID_ARG, "logits is NULL");
  if ((s = check_io(c, false, true)) != TMX_OK) return s;
  (void)hipSetDevice(c->device);
  return run_head(c, y, logits, B, as_stream(stream));
}

tmx_status tmx_model_forward(tmx_ctx* c, const void* emb, float* logits, int B, void* stream) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  tmx_status s;
  if ((s = check_B(c, B)) != TMX_OK) return s;
  if ((s = check_act(c, emb, "emb")) != TMX_OK) return s;
  if (!logits) return fail(c, TMX_ERR_INVALID_ARG, "logits is NULL");
  if ((s = check_io(c, true, true)) != TMX_OK) return s;
  if ((s = check_ready(c)) != TMX_OK) return s;
  (void)hipSetDevice(c->device);
  hipStream_t st = as_stream(stream);
  if ((s = run_tokenize(c, emb, c->io.xbuf, B, st)) != TMX_OK) return s;
  if ((s = tmx_block_stack_forward(c, c->io.xbuf, c->io.ybuf, B, stream)) != TMX_OK) return s;
  return run_head(c, c->io.ybuf, logits, B, st);
}

tmx_status tmx_set_kernel_timing(tmx_ctx* c, int enable) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  if (enable != 0 && enable != 1) return fail(c, TMX_ERR_INVALID_ARG, "enable must be 0 or 1");
  c->timing = enable == 1;
  return TMX_OK;
}

tmx_status tmx_kernel_times(tmx_ctx* c, double* ms, long long* launches, int n) {
  if (!c) return fail(nullptr, TMX_ERR_INVALID_ARG, "ctx is NULL");
  if (n < 0 || ((!ms || !launches) && n > 0)) return fail(c, TMX_ERR_INVALID_ARG, "ms / launches / n invalid");
  (void)hipSetDevice(c->device);
  tmx_status st = TMX_OK;
  for (auto& t : c->pending) {
    float e_ms = 0.f;
    hipError_t e = hipEventSynchronize(t.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&e_ms, t.start, t.end);
    if (e != hipSuccess && st == TMX_OK) st = fail(c, TMX_ERR_DEVICE, "kernel timing: %s", hipGetErrorString(e));
    c->kernel_ms[t.kind] += e_ms;
    c->kernel_launches[t.kind] += 1;
    c->event_pool.push_back(t.start);
    c->event_pool.push_back(t.end);
  }
  c->pending.clear();
  for (int k = 0; k < TMX_KERNEL_KINDS; ++k) {
    if (k < n) {
      ms[k] = c->kernel_ms[k];
      launches[k] = c->kernel_launches[k];
    }
    c->kernel_ms[k] = 0.0;
    c->kernel_launches[k] = 0;
  }
  return st;
}

}  // extern "C"
