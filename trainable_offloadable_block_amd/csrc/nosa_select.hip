// Two-stage block selection (aiwiki "NOSA", How NOSA works; NOSA-1B
// 核心组件揭秘, 核心组件三; l189 article, 2.1).
//
// score_kernel  (pairs x chunk splits): query-aware logits of the GQA group
//   against the compressed keys on MFMA, l = q . c / sqrt(128); per split and
//   head, m = max l, Z = sum exp(l - m); stores e = exp(l - m) per chunk.
// pool_topk_kernel (one workgroup per pair): combines the split statistics
//   into the per-head softmax, sums the group's heads, max-pools the chunks
//   overlapping each block, then stage 1 (top k_q by the query-aware score)
//   and stage 2 (top k_e' eligible by the agnostic score), writes the
//   ascending selection and clears the eligibility of every candidate left
//   out (never re-selected by the agnostic stage).
#include "nosa_internal.h"

namespace nosa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 256;

// MFMA 16x16x32 (bf16 -> fp32) operand mapping used here and in decode:
//  A (16 rows x 32 k): lane l gives row (l % 16), 8 k-values of group l / 16
//  B (32 k x 16 cols): lane l gives col (l % 16), 8 k-values of group l / 16
//  D (16 x 16):        lane l holds rows 4*(l/16) + i, i = 0..3, col l % 16
// Dot products only need A and B to assign the same k to the same
// (lane group, slot), which holds by construction. Rows of A are permuted
// so that, over two tiles, lane group j holds 8 consecutive rows (chunks):
// tile t, A-row r  <->  row 8*(r/4) + 4*t + (r%4) of the 32-row group.
__device__ inline int tile_row(int r, int t) { return 8 * (r >> 2) + 4 * t + (r & 3); }

__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    Dims d, const int32_t *__restrict__ seq_len, const uint16_t *__restrict__ ckey,
    const uint16_t *__restrict__ q, float *__restrict__ ws_e,
    float2 *__restrict__ ws_stats, int c_pad, int n_splits) {
  const int split = blockIdx.x, p = blockIdx.y;
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int C = min(chunks_for(seq_len[b]), d.C_max);
  const int c0 = split * kChunksPerSplit;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
  __shared__ float red_m[4][16], red_z[4][16];
  float2 *stats = ws_stats + (size_t)(p * n_splits + split) * d.G;
  if (c0 >= C) {
    if (threadIdx.x < d.G) stats[threadIdx.x] = make_float2(-INFINITY, 0.0f);
    return;
  }
  bf16x8 qop[4];
  if (h < d.G) {
    const uint16_t *qh = q + ((size_t)b * d.Hq + g * d.G + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qh + 32 * s));
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  const int cg = c0 + 32 * w;
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int chunk = cg + tile_row(l & 15, t);
    uint4 a[4];
    if (chunk < C) {
      const uint16_t *src = ckey + ((size_t)p * d.C_max + chunk) * kHeadDim + 8 * lg;
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const uint4 *>(src + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = make_uint4(0, 0, 0, 0);
    }
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t] = mfma16x16x32(as_bf16x8(a[s]), qop[s], acc[t]);
  }
  // lane (h, lg) now holds head h against chunks cg + 8*lg + m, m = 0..7
  const float scale = 0.08838834764831845f;   // 1/sqrt(128)
  float x[8];
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int c = cg + 8 * lg + m;
    x[m] = c < C ? acc[m >> 2][m & 3] * scale : -INFINITY;
    mx = fmaxf(mx, x[m]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (lg == 0) red_m[w][h] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
  float ev[8];
  float z = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    ev[m] = x[m] == -INFINITY ? 0.0f : expf(x[m] - M);
    z += ev[m];
  }
  z += __shfl_xor(z, 16, 64);
  z += __shfl_xor(z, 32, 64);
  if (lg == 0) red_z[w][h] = z;
  if (h < d.G) {
    float *dst = ws_e + ((size_t)p * d.G + h) * c_pad + cg + 8 * lg;
    if (cg + 8 * lg + 8 <= C) {
      reinterpret_cast<float4 *>(dst)[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
      reinterpret_cast<float4 *>(dst)[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (cg + 8 * lg + m < C) dst[m] = ev[m];
    }
  }
  __syncthreads();
  if (threadIdx.x < d.G) {
    const int hh = threadIdx.x;
    const float Mh = fmaxf(fmaxf(red_m[0][hh], red_m[1][hh]), fmaxf(red_m[2][hh], red_m[3][hh]));
    const float Zh = (red_z[0][hh] + red_z[1][hh]) + (red_z[2][hh] + red_z[3][hh]);
    stats[hh] = make_float2(Mh, Zh);
  }
}

// Exclusive prefix sum over the 256 threads of a workgroup.
__device__ int block_excl_scan(int v, int *sh, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int j = 0; j < kTopkThreads / 64; ++j) {
    if (j < w) base += sh[j];
    tot += sh[j];
  }
  __syncthreads();
  if (total) *total = tot;
  return base + incl - v;
}

// Marks (kind[i] = val) the k items of largest key among keys[0..n); key 0
// means "not eligible"; among equal keys the lower index wins. Radix select
// on 8-bit digits from the top, then one ordered pass for the ties.
__device__ void topk_mark(const uint32_t *keys, int n, int k, uint8_t *kind,
                          uint8_t val, int *hist, int *sh) {
  const int t = threadIdx.x;
  if (k <= 0 || n <= 0) return;
  int cnt = 0;
  for (int i = t; i < n; i += kTopkThreads) cnt += keys[i] != 0u;
  int valid = 0;
  block_excl_scan(cnt, sh, &valid);
  if (valid <= k) {
    for (int i = t; i < n; i += kTopkThreads)
      if (keys[i] != 0u) kind[i] = val;
    __syncthreads();
    return;
  }
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
    for (int i = t; i < n; i += kTopkThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (t < 64) {
      const int c0 = hist[255 - 4 * t], c1 = hist[254 - 4 * t];
      const int c2 = hist[253 - 4 * t], c3 = hist[252 - 4 * t];
      const int s = c0 + c1 + c2 + c3;
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int nb = __shfl_up(incl, o, 64);
        if (t >= o) incl += nb;
      }
      const int excl = incl - s;
      if (excl < rem && rem <= incl) {
        const int r = rem - excl;
        int digit, above = excl;
        if (r <= c0) {
          digit = 255 - 4 * t;
        } else if (r <= c0 + c1) {
          digit = 254 - 4 * t; above += c0;
        } else if (r <= c0 + c1 + c2) {
          digit = 253 - 4 * t; above += c0 + c1;
        } else {
          digit = 252 - 4 * t; above += c0 + c1 + c2;
        }
        sh[4] = digit;
        sh[5] = rem - above;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh[4]) << shift;
    mask |= 0xFFu << shift;
    rem = sh[5];
    __syncthreads();
  }
  // keys above the threshold are in; `rem` threshold-equal keys join them,
  // lowest index first
  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int lo = t * per, hi = min(n, lo + per);
  int eq = 0;
  for (int i = lo; i < hi; ++i) eq += keys[i] == prefix;
  int before = block_excl_scan(eq, sh, nullptr);
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    if (key > prefix) {
      kind[i] = val;
    } else if (key == prefix) {
      if (before < rem) kind[i] = val;
      ++before;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void pool_topk_kernel(
    Dims d, nosa_state st, const float *__restrict__ ws_e,
    const float2 *__restrict__ ws_stats, int c_pad, int n_splits,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
    uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  extern __shared__ __align__(16) uint8_t smem[];
  float *f_sh = reinterpret_cast<float *>(smem);                       // [n_splits][G]
  uint32_t *keys = reinterpret_cast<uint32_t *>(f_sh + n_splits * d.G); // [NB_max]
  uint8_t *kind = reinterpret_cast<uint8_t *>(keys + d.NB_max);         // [NB_max]
  __shared__ int hist[256];
  __shared__ int sh[8];

  const int p = blockIdx.x, t = threadIdx.x;
  const int b = p / d.Hkv;
  const int L = max(0, min(st.seq_len[b], d.max_context));
  int C = chunks_for(L);
  if (C > c_pad) {                      // caller's length bound was too small
    if (t == 0) atomicOr(st.status, NOSA_STATUS_LEN_HINT);
    C = c_pad;
  }
  const int nb = blocks_for(L);
  const int win_lo = max(d.n_sink, nb - d.n_win);
  const int n_cand = max(0, win_lo - d.n_sink);
  const int used = (C + kChunksPerSplit - 1) / kChunksPerSplit;

  // 1. per-split factors exp(m_split - M) / Z of each head's softmax
  if (n_cand > 0 && d.k_q > 0) {
    const int h = t >> 4, j = t & 15;
    if (h < d.G) {
      const float2 *stp = ws_stats + (size_t)p * n_splits * d.G;
      double m = -INFINITY;
      for (int s = j; s < used; s += 16) m = fmax(m, (double)stp[s * d.G + h].x);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
      double z = 0.0;
      for (int s = j; s < used; s += 16) {
        const float2 v = stp[s * d.G + h];
        if (v.y > 0.0f) z += (double)v.y * exp((double)v.x - m);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
      for (int s = j; s < used; s += 16) {
        const float2 v = stp[s * d.G + h];
        f_sh[s * d.G + h] = v.y > 0.0f ? (float)(exp((double)v.x - m) / z) : 0.0f;
      }
    }
  }
  for (int bb = t; bb < nb; bb += kTopkThreads)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);
  __syncthreads();

  // 2. query-aware block score: max over overlapping chunks of the group sum
  if (d.k_q > 0) {
    const float *ep = ws_e + (size_t)p * d.G * c_pad;
    for (int i = t; i < n_cand; i += kTopkThreads) {
      const int bb = d.n_sink + i;
      const int lo = max(0, 4 * bb - 1), hi = min(C, 4 * bb + 4);
      float qb = -INFINITY;
      for (int c = lo; c < hi; ++c) {
        const float *fs = f_sh + (c / kChunksPerSplit) * d.G;
        float a = 0.0f;
        for (int h = 0; h < d.G; ++h) a = fmaf(ep[(size_t)h * c_pad + c], fs[h], a);
        qb = fmaxf(qb, a);
      }
      keys[i] = order_key(qb);
      if (dbg) dbg[(size_t)p * d.NB_max + bb] = qb;
    }
    __syncthreads();
    topk_mark(keys, n_cand, d.k_q, kind + d.n_sink, NOSA_KIND_QUERY, hist, sh);
  }

  // 3. agnostic stage over eligible candidates not taken by stage 1
  if (d.k_e_dyn > 0) {
    const uint32_t *el = st.eligible + (size_t)p * d.elig_words;
    const float *be = st.blk_e + (size_t)p * d.NB_max;
    for (int i = t; i < n_cand; i += kTopkThreads) {
      const int bb = d.n_sink + i;
      const bool elig = (el[bb >> 5] >> (bb & 31)) & 1u;
      keys[i] = (elig && kind[bb] != NOSA_KIND_QUERY) ? order_key(be[bb]) : 0u;
    }
    __syncthreads();
    topk_mark(keys, n_cand, d.k_e_dyn, kind + d.n_sink, NOSA_KIND_AGNOSTIC, hist, sh);
  }

  // 4. ascending selection list
  {
    const int per = (nb + kTopkThreads - 1) / kTopkThreads;
    const int lo = t * per, hi = min(nb, lo + per);
    int cnt = 0;
    for (int bb = lo; bb < hi; ++bb) cnt += kind[bb] != NOSA_KIND_NONE;
    int total = 0;
    int off = block_excl_scan(cnt, sh, &total);
    int32_t *sp = sel + (size_t)p * d.k;
    uint8_t *kp = kind_out ? kind_out + (size_t)p * d.k : nullptr;
    for (int bb = lo; bb < hi; ++bb) {
      if (kind[bb] != NOSA_KIND_NONE && off < d.k) {
        sp[off] = bb;
        if (kp) kp[off] = kind[bb];
        ++off;
      }
    }
    for (int j = total + t; j < d.k; j += kTopkThreads) {
      sp[j] = -1;
      if (kp) kp[j] = NOSA_KIND_NONE;
    }
    if (t == 0) n_sel[p] = min(total, d.k);
  }

  // 5. eligibility: a candidate outside the selection is out for good
  if (n_cand > 0) {
    uint32_t *el = st.eligible + (size_t)p * d.elig_words;
    const int w0 = d.n_sink >> 5, w1 = (win_lo - 1) >> 5;
    for (int wd = w0 + t; wd <= w1; wd += kTopkThreads) {
      uint32_t clear = 0u;
      for (int j = 0; j < 32; ++j) {
        const int bb = wd * 32 + j;
        if (bb >= d.n_sink && bb < win_lo && kind[bb] == NOSA_KIND_NONE) clear |= 1u << j;
      }
      if (clear) el[wd] &= ~clear;
    }
  }
}

}  // namespace

SelectLayout select_layout(const Dims &d, int max_len) {
  SelectLayout s;
  const int C = chunks_for(max_len);
  s.n_splits = C > 0 ? (C + kChunksPerSplit - 1) / kChunksPerSplit : 1;
  s.c_pad = s.n_splits * kChunksPerSplit;
  s.e_off = 0;
  s.stats_off = ((size_t)d.P * d.G * s.c_pad * sizeof(float) + 255) & ~(size_t)255;
  s.bytes = s.stats_off + (((size_t)d.P * s.n_splits * d.G * sizeof(float2) + 255) & ~(size_t)255);
  return s;
}

hipError_t launch_select(const Dims &d, const nosa_state &st, const uint16_t *q,
                         int32_t *sel, int32_t *n_sel, uint8_t *kind, float *dbg,
                         void *ws, const SelectLayout &lay, hipStream_t s) {
  float *ws_e = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.e_off);
  float2 *ws_stats = reinterpret_cast<float2 *>(static_cast<char *>(ws) + lay.stats_off);
  score_kernel<<<dim3(lay.n_splits, d.P), kScoreThreads, 0, s>>>(
      d, st.seq_len, st.ckey, q, ws_e, ws_stats, lay.c_pad, lay.n_splits);
  const size_t lds = (size_t)lay.n_splits * d.G * sizeof(float) +
                     (size_t)d.NB_max * sizeof(uint32_t) + (size_t)d.NB_max;
  pool_topk_kernel<<<dim3(d.P), kTopkThreads, lds, s>>>(
      d, st, ws_e, ws_stats, lay.c_pad, lay.n_splits, sel, n_sel, kind, dbg);
  return hipGetLastError();
}

}  // namespace nosa
