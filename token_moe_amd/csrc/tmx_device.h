// tmx_device.h -- device-side helpers shared by the gfx950 kernels:
// bf16 conversion, the Mix/Revert index map, MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is carried as its 16-bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest, ties to even (finite inputs; the path never makes NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ float silu(float z) {
  // z * sigmoid(z); expf of a large positive argument gives +inf and 1/inf = 0,
  // which is the right limit.
  return z / (1.0f + __expf(-z));
}

// ---------------------------------------------------------------------------
// Position-major view of a [B, T, D] block tensor: the one Mix / Revert
// address map of the library. Every kernel that reads or writes block-layout
// rows by position (the fused MLP's row I/O, the router, the RankMixer token
// mixing, the fp32 path, the debug permutation) computes its offsets with
// the functions below and nothing else.
//
// Mix sub-layer (TokenMixer-Large Eq. 9-11): position p = head h, width
// W = T*dh, element w = t*dh + j lives at X[b, t, h*dh + j]. Revert (Eq.
// 13-15) is the same bijection read the other way, so the mix sub-layer
// reads its input and writes X_rev through this one map.
// Revert sub-layer: position p = token t, width W = D, identity.
//
// offset(b, p, w) = row(b) + pos(p) + col(w): the three parts are separate
// so that a kernel can keep a part that does not change across its units
// (a lane whose column group is fixed computes col() once), and cursor()
// steps col() along a row by a constant stride without a division per step.
// ---------------------------------------------------------------------------
struct RowMap {
  int T, D, dh;   // dh = D / H
  int mix;        // 1: mixed positions, 0: token positions

  __device__ __forceinline__ int64_t row(int64_t b) const { return b * (int64_t)T * D; }
  __device__ __forceinline__ int64_t pos(int p) const { return (int64_t)p * (mix ? dh : D); }
  __device__ __forceinline__ int col(int w) const {
    if (mix) {
      const int t = w / dh;
      return t * D + (w - t * dh);
    }
    return w;
  }
  __device__ __forceinline__ int64_t offset(int64_t b, int p, int w) const { return row(b) + pos(p) + col(w); }

  // col(w0), col(w0 + s), col(w0 + 2s), ... for a stride s > 0
  struct Cursor {
    int seg, j, dh, D;
    __device__ __forceinline__ int col() const { return seg * D + j; }
    __device__ __forceinline__ void advance(int s) {
      j += s;
      while (j >= dh) {
        j -= dh;
        ++seg;
      }
    }
  };
  __device__ __forceinline__ Cursor cursor(int w0) const {
    if (mix) return Cursor{w0 / dh, w0 % dh, dh, D};
    return Cursor{0, w0, 0x7fffffff, 0};
  }
};

// 16-byte vector of 8 bf16
struct alignas(16) bf16v8 {
  uint16_t v[8];
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment layouts (wave64, 8 bf16 = 16 bytes per lane for A and B):
// v_mfma_f32_16x16x32_bf16
//   A (16 x 32, M x K): lane l holds A[l % 16][8*(l/16) + i], i = 0..7
//   B (32 x 16, K x N): lane l holds B[8*(l/16) + i][l % 16]
//   C (16 x 16):        lane l holds C[4*(l/16) + v][l % 16], v = 0..3
// v_mfma_f32_32x32x16_bf16
//   A (32 x 16, M x K): lane l holds A[l % 32][8*(l/32) + i], i = 0..7
//   B (16 x 32, K x N): lane l holds B[8*(l/32) + i][l % 32]
//   C (32 x 32):        lane l holds C[8*(v/4) + 4*(l/32) + v%4][l % 32], v = 0..15
// A packed weight fragment is the 64 x 8 bf16 block a wave loads as B, so
// each lane reads 16 contiguous bytes.
constexpr int FRAG_ELEMS = 512;

}  // namespace tmx
