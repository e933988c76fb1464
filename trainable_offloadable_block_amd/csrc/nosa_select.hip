// Two-stage block selection (aiwiki "NOSA", How NOSA works; NOSA-1B
// 核心组件揭秘, 核心组件三; l189 article, 2.1).
//
// score_kernel  (pairs x chunk splits): query-aware logits of the GQA group
//   against the compressed keys on MFMA, l = q . c / sqrt(128); per split and
//   head, m = max l, Z = sum exp(l - m); stores e = exp(l - m) per chunk.
// pool_topk_kernel (one workgroup per pair): combines the split statistics
//   into the per-head softmax, sums the group's heads, max-pools the chunks
//   overlapping each block, then stage 1 (top k_q by the query-aware score)
//   and stage 2 (top k_e' eligible by the agnostic score), each a wave-level
//   bitonic top-k over 64-candidate chunks merged across waves, writes the
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

// ---- wave-level top-k on 64-bit composite keys --------------------------
// A key is (order_key(score) << 32) | ~block: larger score first, then the
// lower block id, all keys distinct; 0 marks "not a candidate".

// Value of lane (lane ^ MASK): DPP for masks 1 and 2, ds_swizzle (xor within
// 32 lanes) for 4, 8, 16, ds_bpermute for 32.
template <int MASK>
__device__ inline uint32_t xor_lane(uint32_t v) {
  const int x = static_cast<int>(v);
  if constexpr (MASK == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  } else if constexpr (MASK == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  } else if constexpr (MASK < 32) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, 0x1F | (MASK << 10)));
  } else {
    return static_cast<uint32_t>(__shfl_xor(x, MASK, 64));
  }
}

template <int MASK>
__device__ inline uint64_t xor_lane_u64(uint64_t v) {
  const uint32_t lo = xor_lane<MASK>(static_cast<uint32_t>(v));
  const uint32_t hi = xor_lane<MASK>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ inline uint64_t lane_u64(uint64_t v, int src) {
  const int lo = __shfl(static_cast<int>(v & 0xFFFFFFFFu), src, 64);
  const int hi = __shfl(static_cast<int>(v >> 32), src, 64);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// One compare-exchange step of a bitonic network with partner lane ^ J;
// lanes whose (lane & J) == 0 keep the max when `keep_max_low`.
template <int J>
__device__ inline uint64_t cas_step(uint64_t v, bool keep_max_low) {
  const int lane = threadIdx.x & 63;
  const uint64_t o = xor_lane_u64<J>(v);
  const bool lower = (lane & J) == 0;
  return (lower == keep_max_low) ? (v > o ? v : o) : (v < o ? v : o);
}

template <int K>
__device__ inline uint64_t sort_stage(uint64_t v) {
  const bool desc = ((threadIdx.x & 63) & K) == 0;   // direction of this K-block
  if constexpr (K >= 64) v = cas_step<32>(v, desc);
  if constexpr (K >= 32) v = cas_step<16>(v, desc);
  if constexpr (K >= 16) v = cas_step<8>(v, desc);
  if constexpr (K >= 8) v = cas_step<4>(v, desc);
  if constexpr (K >= 4) v = cas_step<2>(v, desc);
  v = cas_step<1>(v, desc);
  return v;
}

// Bitonic sort of one key per lane; afterwards lane i holds the i-th largest.
__device__ inline uint64_t wave_sort_desc(uint64_t v) {
  v = sort_stage<2>(v);
  v = sort_stage<4>(v);
  v = sort_stage<8>(v);
  v = sort_stage<16>(v);
  v = sort_stage<32>(v);
  return sort_stage<64>(v);
}

// Top 64 of two descending-sorted wave lists, sorted descending: the
// element-wise max of a and reversed b is bitonic and holds the 64 largest.
__device__ inline uint64_t wave_merge_desc(uint64_t a, uint64_t b) {
  const uint64_t br = lane_u64(b, 63 - (threadIdx.x & 63));
  uint64_t v = a > br ? a : br;
  v = cas_step<32>(v, true);
  v = cas_step<16>(v, true);
  v = cas_step<8>(v, true);
  v = cas_step<4>(v, true);
  v = cas_step<2>(v, true);
  return cas_step<1>(v, true);
}

__device__ inline uint64_t compose_key(float score, int blk) {
  return (static_cast<uint64_t>(order_key(score)) << 32) |
         static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(blk));
}

__device__ inline int key_block(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFu));
}

// Combines the four waves' sorted top-64 lists and marks the best k blocks
// (kind[b] = val). Called by all threads of the workgroup.
__device__ void finish_topk(uint64_t best, int k, uint8_t *kind, uint8_t val,
                            uint64_t (*top_sh)[64]) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  top_sh[w][lane] = best;
  __syncthreads();
  if (w == 0) {
    const uint64_t b1 = top_sh[1][lane], b2 = top_sh[2][lane], b3 = top_sh[3][lane];
    best = wave_merge_desc(wave_merge_desc(best, b1), wave_merge_desc(b2, b3));
    if (lane < k && best != 0) kind[key_block(best)] = val;
  }
  __syncthreads();
}

// Query-aware score of block bb from the 5 x G chunk weights ev (chunks
// 4bb-1 .. 4bb+3), with the per-split softmax factors f_sh.
__device__ inline float block_qscore(const float (&ev)[5][kMaxGroup], int bb, int C,
                                     const float *f_sh, int G) {
  float qb = -INFINITY;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int c = 4 * bb - 1 + j;
    if (c < 0 || c >= C) continue;
    const float *fs = f_sh + (c / kChunksPerSplit) * G;
    float a = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      if (h < G) a = fmaf(ev[j][h], fs[h], a);
    qb = fmaxf(qb, a);
  }
  return qb;
}

__device__ inline void load_weights(float (&ev)[5][kMaxGroup], const float *ep, int bb, int C,
                                    int c_pad, int G) {
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int c = 4 * bb - 1 + j;
    const bool cin = c >= 0 && c < C;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) ev[j][h] = (cin && h < G) ? ep[(size_t)h * c_pad + c] : 0.0f;
  }
}

__global__ __launch_bounds__(kTopkThreads) void pool_topk_kernel(
    Dims d, nosa_state st, const float *__restrict__ ws_e,
    const float2 *__restrict__ ws_stats, int c_pad, int n_splits,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
    uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  extern __shared__ __align__(16) uint8_t smem[];
  float *f_sh = reinterpret_cast<float *>(smem);                            // [n_splits][G]
  uint32_t *el_sh = reinterpret_cast<uint32_t *>(f_sh + n_splits * d.G);    // [elig_words]
  uint8_t *kind = reinterpret_cast<uint8_t *>(el_sh + d.elig_words);        // [NB_max]
  __shared__ uint64_t top_sh[kTopkThreads / 64][64];
  __shared__ int sh[8];

  const int p = blockIdx.x, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
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
  const bool do_q = d.k_q > 0 && n_cand > 0, do_e = d.k_e_dyn > 0 && n_cand > 0;

  // 0. issue this thread's global loads together: split statistics, the
  // chunk weights and agnostic score of its first candidate, eligibility
  const float *ep = ws_e + (size_t)p * d.G * c_pad;
  const float *be = st.blk_e + (size_t)p * d.NB_max;
  const int i0 = 64 * w + lane, bb0 = d.n_sink + i0;
  const bool have0 = i0 < n_cand;
  float ev[5][kMaxGroup];
  if (do_q) load_weights(ev, ep, have0 ? bb0 : 0, have0 ? C : 0, c_pad, d.G);
  const float e0 = (do_e && have0) ? be[bb0] : 0.0f;
  const int sh_h = t >> 4, sh_j = t & 15;
  float2 stv = make_float2(-INFINITY, 0.0f);
  if (do_q && sh_h < d.G && sh_j < used) stv = ws_stats[((size_t)p * n_splits + sh_j) * d.G + sh_h];
  for (int i = t; i < d.elig_words; i += kTopkThreads)
    el_sh[i] = st.eligible[(size_t)p * d.elig_words + i];
  for (int bb = t; bb < nb; bb += kTopkThreads)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);

  // 1. per-split factors exp(m_split - M) / Z of each head's softmax
  if (do_q && sh_h < d.G) {
    const float2 *stp = ws_stats + (size_t)p * n_splits * d.G;
    double m = stv.x;
    for (int s = sh_j + 16; s < used; s += 16) m = fmax(m, (double)stp[s * d.G + sh_h].x);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
    double z = stv.y > 0.0f ? (double)stv.y * exp((double)stv.x - m) : 0.0;
    for (int s = sh_j + 16; s < used; s += 16) {
      const float2 v = stp[s * d.G + sh_h];
      if (v.y > 0.0f) z += (double)v.y * exp((double)v.x - m);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
    if (sh_j < used) f_sh[sh_j * d.G + sh_h] = stv.y > 0.0f ? (float)(exp((double)stv.x - m) / z) : 0.0f;
    for (int s = sh_j + 16; s < used; s += 16) {
      const float2 v = stp[s * d.G + sh_h];
      f_sh[s * d.G + sh_h] = v.y > 0.0f ? (float)(exp((double)v.x - m) / z) : 0.0f;
    }
  }
  __syncthreads();

  // 2. stage 1: top k_q candidates by the query-aware score (max over the
  // overlapping chunks of the group's softmax sum; heads summed in order, so
  // a chunk shared by two blocks gives both the same value)
  if (do_q) {
    uint64_t best = 0;
    for (int base = 64 * w; base < n_cand; base += kTopkThreads) {   // wave-uniform
      const int i = base + lane, bb = d.n_sink + i;
      if (base != 64 * w) load_weights(ev, ep, i < n_cand ? bb : 0, i < n_cand ? C : 0, c_pad, d.G);
      uint64_t key = 0;
      if (i < n_cand) {
        const float qb = block_qscore(ev, bb, C, f_sh, d.G);
        key = compose_key(qb, bb);
        if (dbg) dbg[(size_t)p * d.NB_max + bb] = qb;
      }
      best = wave_merge_desc(best, wave_sort_desc(key));
    }
    finish_topk(best, d.k_q, kind, NOSA_KIND_QUERY, top_sh);
  }

  // 3. stage 2: top k_e' of the eligible candidates left by stage 1, by the
  // query-agnostic score
  if (do_e) {
    uint64_t best = 0;
    for (int base = 64 * w; base < n_cand; base += kTopkThreads) {   // wave-uniform
      const int i = base + lane, bb = d.n_sink + i;
      uint64_t key = 0;
      if (i < n_cand) {
        const float eb = base == 64 * w ? e0 : be[bb];
        const bool elig = (el_sh[bb >> 5] >> (bb & 31)) & 1u;
        if (elig && kind[bb] != NOSA_KIND_QUERY) key = compose_key(eb, bb);
      }
      best = wave_merge_desc(best, wave_sort_desc(key));
    }
    finish_topk(best, d.k_e_dyn, kind, NOSA_KIND_AGNOSTIC, top_sh);
  }
  __syncthreads();

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
      if (clear) el[wd] = el_sh[wd] & ~clear;
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
                     (size_t)d.elig_words * sizeof(uint32_t) + (size_t)d.NB_max;
  pool_topk_kernel<<<dim3(d.P), kTopkThreads, lds, s>>>(
      d, st, ws_e, ws_stats, lay.c_pad, lay.n_splits, sel, n_sel, kind, dbg);
  return hipGetLastError();
}

}  // namespace nosa
