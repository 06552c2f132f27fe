// tmx_f32.hip -- fp32 sub-layer (dense per-token SwiGLU or Sparse-Pertoken
// MoE) for fp32 contexts.  One workgroup per (sample, position); plain fp32
// FMA arithmetic, weights in their logical row-major layout.  fp32 shapes
// are small (the tiny dense workload is launch-latency bound), so this path
// favours generality: any W, hidden, E and top_k.
#include "tmx_internal.h"

namespace tmx {

namespace {

constexpr int F_NT = 128;

__device__ float block_sum(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < F_NT / 64; ++i) s += red[i];
  return s;
}

// U = silu(x @ Wg) * (x @ Wu) for one SwiGLU (TokenMixer-Large Eq. 17-18)
__device__ void hidden_f32(const float* xs, int W, int h, const float* wu, const float* wg, float* U) {
  for (int j = threadIdx.x; j < h; j += F_NT) {
    float g = 0.f, u = 0.f;
    for (int i = 0; i < W; ++i) {
      g = fmaf(xs[i], wg[(size_t)i * h + j], g);
      u = fmaf(xs[i], wu[(size_t)i * h + j], u);
    }
    U[j] = g / (1.0f + expf(-g)) * u;
  }
}

__global__ __launch_bounds__(F_NT) void f32_sublayer_kernel(const F32Args a) {
  extern __shared__ float sm[];
  const int W = a.W;
  const int hmax = max(a.hidden, max(a.expert_hidden, a.shared_hidden));
  float* xs = sm;               // [W]
  float* acc = xs + W;          // [W]
  float* U = acc + W;           // [hmax]
  float* lg = U + hmax;         // [E]
  float* red = lg + max(a.E, 1);  // [F_NT/64]
  __shared__ int sel[64];
  __shared__ float selg[64];

  const int b = blockIdx.x / a.P, p = blockIdx.x % a.P;
  const int tid = threadIdx.x;

  float ss = 0.f;
  for (int w = tid; w < W; w += F_NT) {
    const float v = a.x[a.map.offset(b, p, w)];
    xs[w] = v;
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rinv = 1.0f / sqrtf(ss / (float)W + a.eps);
  for (int w = tid; w < W; w += F_NT) {
    xs[w] = xs[w] * rinv * a.gain[w];
    acc[w] = 0.f;
  }
  __syncthreads();

  if (a.E == 0) {
    hidden_f32(xs, W, a.hidden, a.w_up + (size_t)p * W * a.hidden, a.w_gate + (size_t)p * W * a.hidden, U);
    __syncthreads();
    const float* wd = a.w_down + (size_t)p * a.hidden * W;
    for (int w = tid; w < W; w += F_NT) {
      float o = 0.f;
      for (int j = 0; j < a.hidden; ++j) o = fmaf(U[j], wd[(size_t)j * W + w], o);
      acc[w] = o;
    }
  } else {
    // router (Eq. 19, 21): logits, softmax over all E, top_k by (-logit, index)
    const float* wr = a.w_router + (size_t)p * W * a.E;
    for (int e = tid; e < a.E; e += F_NT) {
      float l = 0.f;
      for (int i = 0; i < W; ++i) l = fmaf(xs[i], wr[(size_t)i * a.E + e], l);
      lg[e] = l;
    }
    __syncthreads();
    if (tid == 0) {
      float m = lg[0];
      for (int e = 1; e < a.E; ++e) m = fmaxf(m, lg[e]);
      float den = 0.f;
      for (int e = 0; e < a.E; ++e) den += expf(lg[e] - m);
      uint64_t taken[4] = {0, 0, 0, 0};
      for (int s = 0; s < a.top_k; ++s) {
        int be = -1;
        float bl = 0.f;
        for (int e = 0; e < a.E; ++e) {
          if ((taken[e >> 6] >> (e & 63)) & 1ull) continue;
          if (be < 0 || lg[e] > bl) {
            be = e;
            bl = lg[e];
          }
        }
        taken[be >> 6] |= 1ull << (be & 63);
        sel[s] = be;
        selg[s] = a.alpha * (expf(bl - m) / den);
        const size_t o = ((size_t)b * a.P + p) * a.top_k + s;
        if (a.idx) a.idx[o] = be;
        if (a.gate_out) a.gate_out[o] = selg[s];
      }
    }
    __syncthreads();
    if (a.route_only) return;
    const int he = a.expert_hidden, hs = a.shared_hidden;
    for (int s = 0; s < a.top_k; ++s) {
      const size_t pe = (size_t)p * a.E + sel[s];
      hidden_f32(xs, W, he, a.e_up + pe * W * he, a.e_gate + pe * W * he, U);
      __syncthreads();
      const float* wd = a.e_down + pe * he * W;
      const float g = selg[s];
      for (int w = tid; w < W; w += F_NT) {
        float o = 0.f;
        for (int j = 0; j < he; ++j) o = fmaf(U[j], wd[(size_t)j * W + w], o);
        acc[w] += g * o;
      }
      __syncthreads();
    }
    hidden_f32(xs, W, hs, a.s_up + (size_t)p * W * hs, a.s_gate + (size_t)p * W * hs, U);
    __syncthreads();
    const float* wd = a.s_down + (size_t)p * hs * W;
    for (int w = tid; w < W; w += F_NT) {
      float o = 0.f;
      for (int j = 0; j < hs; ++j) o = fmaf(U[j], wd[(size_t)j * W + w], o);
      acc[w] += o;
    }
  }
  __syncthreads();
  for (int w = tid; w < W; w += F_NT) {
    const int64_t off = a.map.offset(b, p, w);
    float v = acc[w] + a.resid[off];
    if (a.extra) v += a.extra[off];
    a.out[off] = v;
  }
}

}  // namespace

hipError_t launch_f32_sublayer(const F32Args& a, hipStream_t s) {
  const int hmax = std::max(a.hidden, std::max(a.expert_hidden, a.shared_hidden));
  const size_t shmem = sizeof(float) * (2 * (size_t)a.W + hmax + std::max(a.E, 1) + F_NT / 64);
  hipLaunchKernelGGL(f32_sublayer_kernel, dim3(a.B * a.P), dim3(F_NT), shmem, s, a);
  return hipGetLastError();
}

}  // namespace tmx
