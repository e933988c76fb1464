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

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// bf16 round-to-nearest-even of a float64 value, computed from its bits in
// one step (no intermediate float32 rounding). Handles zeros, subnormal
// results (bf16 shares float32's exponent range: step 2^-133 below 2^-126)
// and overflow to infinity; NaN stays NaN.
__host__ __device__ inline uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
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

// bf16 round-to-nearest-even of the mean of 32 bf16 values (bit patterns
// get(0) .. get(31)), from their exact sum, for any spread of magnitudes
// (NOSA-1B 核心组件揭秘, 核心组件一: the compressed key is the mean of a
// 32-token window). A bf16 value is an 8-bit integer times 2^(E' - 134) with
// E' = max(E, 1) for exponent field E. The float64 sum of 32 of them is
// exact when their E' span at most 40 binades (the sum needs span + 8 + 5
// bits <= 53); a wider span, which no key of a normal range reaches, is
// summed exactly as integers in 320 bits. Infinities and NaNs keep the
// float64 sum's result.
__host__ __device__ inline void add_shifted_u320(uint64_t (&acc)[5], uint64_t m, int sh) {
  const int w = sh >> 6, o = sh & 63;
  const uint64_t lo = m << o, hi = o ? (m >> (64 - o)) : 0;
  uint64_t carry = 0;
  for (int i = 0; i < 5; ++i) {
    const uint64_t x = i == w ? lo : (i == w + 1 ? hi : 0);
    const uint64_t s = acc[i] + x;
    const uint64_t s2 = s + carry;
    carry = (s < x) | (s2 < carry);
    acc[i] = s2;
  }
}

// Bits [lo, lo + n) of a 320-bit value, n <= 64, lo >= 0.
__host__ __device__ inline uint64_t bits_u320(const uint64_t (&a)[5], int lo, int n) {
  const int w = lo >> 6, o = lo & 63;
  uint64_t v = a[w] >> o;
  if (o && w + 1 < 5) v |= a[w + 1] << (64 - o);
  return n >= 64 ? v : (v & ((1ull << n) - 1));
}

template <typename Get>
__host__ __device__ uint16_t mean32_bf16_wide(Get get) {
  uint64_t pos[5] = {0, 0, 0, 0, 0}, neg[5] = {0, 0, 0, 0, 0};
  for (int j = 0; j < kPoolKernel; ++j) {
    const uint16_t v = get(j);
    const int E = (v >> 7) & 0xff;
    const uint64_t m = (E ? 128u : 0u) + (v & 0x7fu);
    if (m == 0) continue;
    // |v| = m * 2^(E' - 134) = m * 2^(sh - 133), sh = E' - 1 in [0, 253]
    if (v & 0x8000u) add_shifted_u320(neg, m, (E > 1 ? E : 1) - 1);
    else add_shifted_u320(pos, m, (E > 1 ? E : 1) - 1);
  }
  // D = |pos - neg|: sum = +-D * 2^-133, mean = +-D * 2^-138
  bool negative = false;
  for (int i = 4; i >= 0; --i) {
    if (pos[i] != neg[i]) { negative = neg[i] > pos[i]; break; }
  }
  uint64_t D[5];
  const uint64_t(&x)[5] = negative ? neg : pos;
  const uint64_t(&y)[5] = negative ? pos : neg;
  uint64_t borrow = 0;
  for (int i = 0; i < 5; ++i) {
    const uint64_t t = x[i] - y[i];
    const uint64_t b1 = x[i] < y[i];
    D[i] = t - borrow;
    borrow = b1 | (t < borrow);
  }
  int h = -1;                                   // top set bit of D
  for (int i = 4; i >= 0 && h < 0; --i)
    if (D[i]) h = 64 * i + 63 - __builtin_clzll(D[i]);
  if (h < 0) return 0;                          // the exact mean is zero
  const uint16_t sign = negative ? 0x8000u : 0u;
  // mean in [2^(h-138), 2^(h-137)): bf16 exponent field h - 11
  int be = h - 11;
  const int drop = be >= 1 ? h - 7 : 5;         // normal: 8 kept bits; else quantum 2^-133
  if (be < 1) be = 0;
  uint64_t kept = bits_u320(D, drop, 64);
  const bool half = bits_u320(D, drop - 1, 1) != 0;
  bool sticky = false;
  for (int i = 0; i < 5 && 64 * i < drop - 1; ++i) {
    const int n = drop - 1 - 64 * i;            // bits of word i below the half bit
    sticky |= (n >= 64 ? D[i] : (D[i] & ((1ull << n) - 1))) != 0;
  }
  if (half && (sticky || (kept & 1))) kept += 1;
  uint32_t bits;
  if (be == 0) {
    bits = static_cast<uint32_t>(kept);         // a carry reaches the smallest normal
  } else {
    if (kept >> 8) { kept >>= 1; be += 1; }
    if (be >= 255) return sign | 0x7F80u;
    bits = (static_cast<uint32_t>(be) << 7) | static_cast<uint32_t>(kept & 0x7f);
  }
  return sign | static_cast<uint16_t>(bits);
}

template <typename Get>
__host__ __device__ inline uint16_t mean32_bf16(Get get) {
  double sum = 0.0;
  int emax = 0, emin = 255;
  bool special = false;
  for (int j = 0; j < kPoolKernel; ++j) {
    const uint16_t v = get(j);
    sum += (double)bf16_to_f32(v);
    const int E = (v >> 7) & 0xff;
    special |= E == 0xff;
    if (v & 0x7fffu) {
      const int e = E > 1 ? E : 1;
      emax = e > emax ? e : emax;
      emin = e < emin ? e : emin;
    }
  }
  if (special || emax - emin <= 40) return f64_to_bf16_rne(sum * (1.0 / kPoolKernel));
  return mean32_bf16_wide(get);
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

// Blocks per pair in the KV pool, the host store and the token-score rows:
// NB_max, or NB_max + 1 when NB_max is a multiple of 129. Every pair's
// region starts at p times this stride, and the decode's workgroups read
// the same block offsets of many pairs at once. At strides of 258 and 516
// blocks (2^23 + 2^16 and 2^24 + 2^17 bytes) those reads crowded part of
// the HBM channels: the 16K decode launch (4 layers, 64 pairs) ran 29.7 and
// 29.2 us, against 26.1-26.6 us at 257, 259-288, 320, 321, 384, 385, 513 and
// 514 blocks, and 26.4 and 27.2 us with the extra block (387 and 645 blocks
// ran 27.1 and 27.0 us, 388 blocks 26.4 us).
__host__ __device__ inline int kv_blocks_per_pair(int nb_max) {
  return nb_max % 129 == 0 ? nb_max + 1 : nb_max;
}

// Device-side launch parameters shared by the kernels.
struct Dims {
  int B, Hq, Hkv, G, P;           // P = B * Hkv pairs
  int max_context, tok_stride, C_max, NB_max, elig_words;
  int NB_kv;       // blocks per pair in the KV pool and host store (kv_blocks_per_pair)
  int n_sink, n_win, k, k_q, k_e_dyn;
  int offload, bias;
  int pool_small;  // 1: a pair with at most 256 candidates finishes with one per thread
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
