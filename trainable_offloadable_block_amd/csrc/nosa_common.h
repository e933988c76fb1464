// Shared device helpers for the NOSA HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nosa.h"

namespace nosa {

constexpr int kHeadDim = 128;
constexpr int kBlock = 64;
constexpr int kPoolKernel = 32;
constexpr int kPoolStride = 16;
constexpr int kBlockElems = 2 * kBlock * kHeadDim;   // K part + V part, bf16
constexpr int kMaxGroup = 16;
constexpr int kMaxK = 128;
constexpr int kMaxContext = 1 << 18;   // 262144 tokens

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__host__ __device__ inline int chunks_for(int L) {
  return L < kPoolKernel ? 0 : (L - kPoolKernel) / kPoolStride + 1;
}
__host__ __device__ inline int blocks_for(int L) {
  return (L + kBlock - 1) / kBlock;
}

// Element offset of (token, dim) inside a block's V part: 1 KiB tiles
// [2 halves][8 dim tiles][4 token groups][16 dims][8 tokens], so that one
// 16-byte load per lane of a wave fetches one whole tile, already in the
// shape of a 16x16x32 MFMA operand (16 dims x 32 tokens of one half).
__host__ __device__ inline int v_index(int tok, int dim) {
  return ((((tok >> 5) * 8 + (dim >> 4)) * 4 + ((tok >> 3) & 3)) * 16 + (dim & 15)) * 8 + (tok & 7);
}

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// bf16 round-to-nearest-even of a float64 value, computed from its bits in
// one step (no intermediate float32 rounding). Handles zeros, subnormal
// results (bf16 shares float32's exponent range: step 2^-133 below 2^-126)
// and overflow to infinity; NaN stays NaN.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
  int e = static_cast<int>((u >> 52) & 0x7ff);
  uint64_t frac = u & 0xFFFFFFFFFFFFFull;
  if (e == 0x7ff) return sign | (frac ? 0x7FC0u : 0x7F80u);
  if (e == 0) return sign;  // float64 subnormals are far below bf16's range
  // value = m * 2^(e - 1075) with the 53-bit significand m
  uint64_t m = frac | (1ull << 52);
  int unbiased = e - 1023;            // 2^unbiased <= |x| < 2^(unbiased+1)
  // bf16 exponent field for this magnitude, and how many of m's low bits
  // fall below bf16's last kept bit
  int be = unbiased + 127;
  int drop;                            // bits of m dropped
  if (be >= 1) {
    drop = 52 - 7;                     // keep 8 significant bits
  } else {
    // subnormal result: quantum 2^-133, i.e. drop down to that weight
    drop = 52 - 7 + (1 - be);
    be = 0;
  }
  if (drop > 63) return sign;          // far below the smallest subnormal
  uint64_t kept = m >> drop;
  uint64_t rem = m & ((1ull << drop) - 1);
  uint64_t half = 1ull << (drop - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  uint32_t bits;
  if (be == 0) {
    bits = static_cast<uint32_t>(kept);           // may carry into 0x80
  } else {
    // kept holds 1.xxxxxxx (8 bits) or 10.0000000 after a carry
    if (kept >> 8) { kept >>= 1; be += 1; }
    if (be >= 255) return sign | 0x7F80u;
    bits = (static_cast<uint32_t>(be) << 7) | static_cast<uint32_t>(kept & 0x7f);
  }
  return sign | static_cast<uint16_t>(bits);
}

// float -> bf16 round-to-nearest-even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Order-preserving map float -> uint32 (larger float -> larger key); never 0
// for a non-NaN float, so 0 can mark "not a candidate".
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float softplus_f32(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Device-side launch parameters shared by the kernels.
struct Dims {
  int B, Hq, Hkv, G, P;           // P = B * Hkv pairs
  int max_context, tok_stride, C_max, NB_max, elig_words;
  int n_sink, n_win, k, k_q, k_e_dyn;
  int offload, bias;
};

// This workgroup's (x, y) in a 2-D grid whose rows (one pair's workgroups,
// x fastest) should share an XCD: the hardware deals workgroups to the 8
// XCDs round-robin by linear id L, so unit (L % 8) * (total / 8) + L / 8
// keeps each run of total / 8 consecutive units on XCD L % 8 (when total is
// a multiple of 8; otherwise the ids are kept). Only placement depends on
// it: the kernels' cross-workgroup traffic is device-coherent either way.
__device__ inline void grid_unit(int &x, int &y) {
  const int nx = gridDim.x, total = nx * gridDim.y;
  int L = blockIdx.x + nx * blockIdx.y;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  x = L % nx;
  y = L / nx;
}

}  // namespace nosa
