// Sparse decode attention over the selected blocks (NOSA-1B 核心组件揭秘,
// 解码阶段如何只用 64 个 KV 块; aiwiki "NOSA", How NOSA works: the eviction
// score enters the logits as an additive bias; l189 article, 2.1, eq. 8).
//
// decode_splitk_kernel: grid (splits, pairs), 4 waves. Each wave walks whole
//   64-token blocks of its split; per 32-token half it computes the group's
//   logits S^T = K Q^T on MFMA (16 query rows padded to the 16x16x32 shape),
//   an online softmax in the log2 domain, and O^T += V^T P^T on MFMA with P
//   split into bf16 hi + lo parts (P alone in bf16 would cost ~1e-3 relative
//   error). The 4 waves merge in LDS; one partial (m, l, o) per split.
// decode_combine_kernel: merges the split partials and normalises.
#include "nosa_internal.h"

namespace nosa {
namespace {

constexpr int kDecThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline int tile_row(int r, int t) { return 8 * (r >> 2) + 4 * t + (r & 3); }

__device__ inline uint4 ldg16(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

__global__ __launch_bounds__(kDecThreads, 2) void decode_splitk_kernel(
    Dims d, const int32_t *__restrict__ seq_len, const uint16_t *__restrict__ q,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ phys,
    const int32_t *__restrict__ n_sel, const uint16_t *__restrict__ kv,
    int slots_per_pair, const float *__restrict__ tok_s,
    float *__restrict__ ws_o, float2 *__restrict__ ws_ml, int bps, int n_splits,
    uint32_t *status) {
  const int split = blockIdx.x, p = blockIdx.y;
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
  const int L = seq_len[b];
  const int ns = max(0, min(n_sel[p], d.k));
  const int e0 = split * bps, e1 = min(ns, e0 + bps);

  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ float sm_o[4][16][kHeadDim + 4];

  bf16x8 qop[4];
  if (h < d.G) {
    const uint16_t *qh = q + ((size_t)b * d.Hq + g * d.G + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(ldg16(qh + 32 * s));
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  const float qscale = 0.08838834764831845f * kLog2e;   // log2(e) / sqrt(128)
  const float bscale = d.bias ? kLog2e : 0.0f;
  const float *tsp = tok_s + (size_t)p * d.tok_stride;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int e = e0 + w; e < e1; e += 4) {
    const int blk = sel[(size_t)p * d.k + e];
    const int slot = phys[(size_t)p * d.k + e];
    if (blk < 0 || blk >= d.NB_max || slot < 0 || slot >= slots_per_pair) {
      if (l == 0) atomicOr(status, NOSA_STATUS_BAD_SEL);
      continue;
    }
    const uint16_t *kb = kv + ((size_t)p * slots_per_pair + slot) * kBlockElems;
    const uint16_t *vb = kb + kBlock * kHeadDim;
    const int tok0 = blk * kBlock;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // issue this half's loads: K rows, V^T rows, eviction scores
      uint4 ka[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t *kr = kb + (32 * half + tile_row(h, t)) * kHeadDim + 8 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = ldg16(kr + 32 * s);
      }
      uint4 va[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        va[dt] = ldg16(vb + (16 * dt + h) * kBlock + 32 * half + 8 * lg);
      const int key0 = tok0 + 32 * half + 8 * lg;   // this lane's 8 keys
      if (tok0 + 32 * half + 32 > L) {
        // partial block: zero V of keys past L so that stale or uninitialised
        // cache bytes cannot reach the sum (their probabilities are 0)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          u16x8 v = __builtin_bit_cast(u16x8, va[dt]);
#pragma unroll
          for (int m = 0; m < 8; ++m)
            if (key0 + m >= L) v[m] = 0;
          va[dt] = __builtin_bit_cast(uint4, v);
        }
      }
      const float4 s0 = *reinterpret_cast<const float4 *>(tsp + key0);
      const float4 s1 = *reinterpret_cast<const float4 *>(tsp + key0 + 4);
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};

      f32x4 acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t] = mfma16x16x32(as_bf16x8(ka[t][s]), qop[s], acc[t]);
      }
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float lg2 = acc[m >> 2][m & 3] * qscale + sv[m] * bscale;
        x[m] = (key0 + m) < L ? lg2 : -INFINITY;
        mx = fmaxf(mx, x[m]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) continue;            // nothing valid yet
      const float alpha = exp2f(m_run - m_new);    // 0 when m_run = -inf
      m_run = m_new;
      float psum = 0.0f;
      uint16_t phi[8], plo[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float pm = exp2f(x[m] - m_new);
        psum += pm;
        const uint16_t hi = f32_to_bf16_rne(pm);
        phi[m] = hi;
        plo[m] = f32_to_bf16_rne(pm - bf16_to_f32(hi));
      }
      l_run = l_run * alpha + psum;
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, u16x8{phi[0], phi[1], phi[2], phi[3],
                                                          phi[4], phi[5], phi[6], phi[7]});
      const bf16x8 blo = __builtin_bit_cast(bf16x8, u16x8{plo[0], plo[1], plo[2], plo[3],
                                                          plo[4], plo[5], plo[6], plo[7]});
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        o[dt] *= alpha;
        o[dt] = mfma16x16x32(as_bf16x8(va[dt]), bhi, o[dt]);
        o[dt] = mfma16x16x32(as_bf16x8(va[dt]), blo, o[dt]);
      }
    }
  }
  // lane (h, lg): head h's running max, its keys' partial sum, and
  // O^T[16*dt + 4*lg + i][h]
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lg == 0) {
    sm_m[w][h] = m_run;
    sm_l[w][h] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][h][16 * dt + 4 * lg + i] = o[dt][i];
  __syncthreads();
  const size_t part = (size_t)p * n_splits + split;
  for (int idx = threadIdx.x; idx < d.G * kHeadDim; idx += kDecThreads) {
    const int hh = idx / kHeadDim, dim = idx % kHeadDim;
    const float M = fmaxf(fmaxf(sm_m[0][hh], sm_m[1][hh]), fmaxf(sm_m[2][hh], sm_m[3][hh]));
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float f = exp2f(sm_m[ww][hh] - M);
        acc += f * sm_o[ww][hh][dim];
        lsum += f * sm_l[ww][hh];
      }
    }
    ws_o[(part * d.G + hh) * kHeadDim + dim] = acc;
    if (dim == 0) ws_ml[part * d.G + hh] = make_float2(M, lsum);
  }
}

// grid (P), block 256: out[b][g*G + h][dim] = sum_s w_s o_s / sum_s w_s l_s
__global__ __launch_bounds__(kDecThreads) void decode_combine_kernel(
    Dims d, const float *__restrict__ ws_o, const float2 *__restrict__ ws_ml,
    int n_splits, float *__restrict__ out) {
  const int p = blockIdx.x;
  const int b = p / d.Hkv, g = p % d.Hkv;
  for (int idx = threadIdx.x; idx < d.G * kHeadDim; idx += kDecThreads) {
    const int hh = idx / kHeadDim, dim = idx % kHeadDim;
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, ws_ml[((size_t)p * n_splits + s) * d.G + hh].x);
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
      for (int s = 0; s < n_splits; ++s) {
        const size_t part = (size_t)p * n_splits + s;
        const float2 ml = ws_ml[part * d.G + hh];
        const float f = exp2f(ml.x - M);
        acc += f * ws_o[(part * d.G + hh) * kHeadDim + dim];
        lsum += f * ml.y;
      }
    }
    out[((size_t)b * d.Hq + g * d.G + hh) * kHeadDim + dim] = lsum > 0.0f ? acc / lsum : 0.0f;
  }
}

}  // namespace

DecodeLayout decode_layout(const Dims &d) {
  DecodeLayout lay;
  int bps = 4;
  // enough workgroups to cover the chip about twice, whole waves per block
  while (bps < 16 && (long)d.P * ((d.k + 2 * bps - 1) / (2 * bps)) >= 1024) bps *= 2;
  if (const char *env = getenv("NOSA_DECODE_BPS")) {
    const int v = atoi(env);
    if (v >= 1 && v <= 64) bps = v;
  }
  lay.blocks_per_split = bps;
  lay.n_splits = (d.k + bps - 1) / bps;
  lay.o_off = 0;
  const size_t parts = (size_t)d.P * lay.n_splits * d.G;
  lay.ml_off = (parts * kHeadDim * sizeof(float) + 255) & ~(size_t)255;
  lay.bytes = lay.ml_off + ((parts * sizeof(float2) + 255) & ~(size_t)255);
  return lay;
}

hipError_t launch_decode(const Dims &d, const nosa_state &st, const uint16_t *q,
                         const int32_t *sel, const int32_t *phys,
                         const int32_t *n_sel, float *out, void *ws,
                         const DecodeLayout &lay, hipStream_t s) {
  float *ws_o = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.o_off);
  float2 *ws_ml = reinterpret_cast<float2 *>(static_cast<char *>(ws) + lay.ml_off);
  const int slots = d.offload ? d.k + 1 : d.NB_max;
  decode_splitk_kernel<<<dim3(lay.n_splits, d.P), kDecThreads, 0, s>>>(
      d, st.seq_len, q, sel, phys, n_sel, st.kv_dev, slots, st.tok_s, ws_o, ws_ml,
      lay.blocks_per_split, lay.n_splits, st.status);
  decode_combine_kernel<<<dim3(d.P), kDecThreads, 0, s>>>(d, ws_o, ws_ml, lay.n_splits, out);
  return hipGetLastError();
}

}  // namespace nosa
