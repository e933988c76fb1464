// Layer-ahead block selection with a forecast head (SparDA: aliyun article,
// 解耦选块与注意力计算 and 轻量化设计与训练; aiwiki "NOSA", Adoption in
// SparDA). While layer l runs, a forecast head of layer l (one per KV group)
// is matched against layer l+1's compressed keys to pick layer l+1's
// query-aware blocks, so layer l+1's delta fetch can start a layer early.
//
// forecast_select_kernel (scoring workgroups x pairs), one launch, run before the
// step's token is appended to the layer, for the length seq_len + 1 that
// token gives it:
//  - every workgroup scores its splits of the chunks that exist: the plain
//    logit f . c / sqrt(128) of the pair's forecast head on MFMA (one B
//    column of the 16x16x32 shape), with neither a softmax nor a sum over
//    heads, published with device-coherent stores;
//  - the pair's last workgroup max-pools the logits over the chunks
//    overlapping each candidate block and runs NOSA's stages: the k_q
//    candidates of highest forecast score, then the k_e' eligible others of
//    highest agnostic score, under the never-reselect rule. Every candidate
//    block's chunks exist before the append (the window holds at least two
//    blocks), so nothing waits for the coming token.
#include <algorithm>

#include "nosa_select_dev.h"

namespace nosa {
namespace {

// Split `split` of pair p: the forecast logits of chunks [c0, c0 + 128) ∩
// [0, C) into ws_l[p][c] (device-coherent stores).
__device__ __forceinline__ void forecast_score(int C, const ScoreIn &in, float *ws_l, int c_pad,
                                               int split, int p) {
  const int c0 = split * kChunksPerSplit;
  if (c0 >= C) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
  const int cg = c0 + 32 * w;
  extern __shared__ __align__(16) uint8_t score_keys[];
  uint4 *ks = reinterpret_cast<uint4 *>(score_keys);
  keys_to_lds(in, ks, -1);
  __syncthreads();
  uint4 kv[2][4];
  keys_from_lds(ks, kv);
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc[t] = mfma16x16x32(as_bf16x8(kv[t][s]), as_bf16x8(in.qv[s]), acc[t]);
  }
  // lane (0, lg) holds the forecast head against chunks cg + 8*lg + m: two
  // runs of 4 contiguous logits, each one 16-byte device-coherent store when
  // all 4 chunks exist (a run crossing C is written element by element)
  if (h == 0) {
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(ws_l + (size_t)p * c_pad, (uint32_t)c_pad * 4);
    const float sc = 0.08838834764831845f;   // 1 / sqrt(128)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = cg + 8 * lg + 4 * t;
      if (c + 4 <= C) {
        const float4 v = make_float4(acc[t][0] * sc, acc[t][1] * sc, acc[t][2] * sc, acc[t][3] * sc);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), lr, 4 * c, 0,
                                               kCoherent);
      } else {
        float *dst = ws_l + (size_t)p * c_pad + c;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c + i < C) put(&dst[i], acc[t][i] * sc);
      }
    }
  }
}

// Pooling and both stages for pair p by its last workgroup; L_now is the
// length before the coming append.
__device__ __forceinline__ void pool_forecast(const Dims &d, const nosa_state &st, int L_now,
                                              const float *ws_l, int c_pad, int32_t *sel,
                                              int32_t *n_sel, uint8_t *kind_out, float *dbg,
                                              int p) {
  extern __shared__ __align__(16) uint8_t smem[];
  float *a_sh = reinterpret_cast<float *>(smem);                            // [c_pad]
  uint32_t *el_sh = reinterpret_cast<uint32_t *>(a_sh + c_pad);             // [elig_words]
  uint8_t *kind = reinterpret_cast<uint8_t *>(el_sh + d.elig_words);        // [NB_max]
  __shared__ TopkLds tk;
  const int t = threadIdx.x;

  // 0. loads bounded by the buffers' extents, issued together: the first
  // batch of logits, candidate t's agnostic score
  const int n4_ext = c_pad / 4;
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(ws_l + (size_t)p * c_pad, (uint32_t)c_pad * 4);
  float4 lb[kLoadBatch];
#pragma unroll
  for (int u = 0; u < kLoadBatch; ++u) {
    const int k4 = t + kTopkThreads * u;
    lb[u] = k4 < n4_ext ? load4_coherent(lr, 16 * k4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float *be = st.blk_e + (size_t)p * d.NB_max;
  const float e0_raw = d.n_sink + t < d.NB_max ? get(&be[d.n_sink + t]) : 0.0f;

  const int L = max(0, min(L_now, d.max_context));
  const int L_next = min(L + 1, d.max_context);
  int C = min(chunks_for(L), d.C_max);
  if (C > c_pad) {                      // caller's length bound was too small
    if (t == 0) atomicOr(st.status, NOSA_STATUS_LEN_HINT);
    C = c_pad;
  }
  const int nb = blocks_for(L_next);
  const int win_lo = max(d.n_sink, nb - d.n_win);
  const int n_cand = max(0, win_lo - d.n_sink);
  const bool do_q = d.k_q > 0 && n_cand > 0, do_e = d.k_e_dyn > 0 && n_cand > 0;
  const float e0 = (do_e && t < n_cand) ? e0_raw : 0.0f;

  for (int i = t; i < d.elig_words; i += kTopkThreads)
    el_sh[i] = st.eligible[(size_t)p * d.elig_words + i];
  for (int bb = t; bb < nb; bb += kTopkThreads)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);
  topk_lds_init(tk);
  // 1. the logits into LDS (entries at and past C are never read)
  if (do_q) {
    const int n4 = (C + 3) / 4;
    for (int k0 = 0; k0 < n4; k0 += kTopkThreads * kLoadBatch) {      // uniform
      if (k0 > 0) {
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int k4 = k0 + t + kTopkThreads * u;
          lb[u] = k4 < n4 ? load4_coherent(lr, 16 * k4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int k4 = k0 + t + kTopkThreads * u;
        if (k4 < n4) reinterpret_cast<float4 *>(a_sh)[k4] = lb[u];
      }
    }
  }
  __syncthreads();
  finish_select(d, st, p, nb, win_lo, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, sel,
                n_sel, kind_out, dbg, tk);
}

__global__ __launch_bounds__(kScoreThreads) void forecast_select_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ f, float *ws_l, int32_t *ws_count,
    int c_pad, int n_splits, int subs, int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
    uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  int wg, p;
  grid_unit_x_major(wg, p);
  __shared__ int sm_last;
  Dims df = d;                       // f is [B][Hkv][128]: a group of one head
  df.G = 1;
  df.Hq = d.Hkv;
  const int L = max(0, min(st.seq_len[p / d.Hkv], d.max_context));
  const int C = min(min(chunks_for(L), d.C_max), c_pad);
  for (int j = 0; j < subs; ++j) {                 // uniform: this workgroup's splits
    const int split = wg * subs + j;
    if (split >= n_splits) break;
    if (j > 0) __syncthreads();                    // the last split's staged keys are read
    ScoreIn in;
    score_load(df, st.ckey, f, split, p, in);
    forecast_score(C, in, ws_l, c_pad, split, p);
  }
  __builtin_amdgcn_s_waitcnt(0);          // this thread's stores have landed
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(&ws_count[p], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (int)gridDim.x - 1;
  __syncthreads();
  if (!sm_last) return;
  pool_forecast(d, st, L, ws_l, c_pad, sel, n_sel, kind_out, dbg, p);
  if (threadIdx.x == 0) __hip_atomic_store(&ws_count[p], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_select_forecast(const Dims &d, const nosa_state &st, const uint16_t *f,
                                  int32_t *sel, int32_t *n_sel, uint8_t *kind, float *dbg,
                                  void *ws, const SelectLayout &lay, hipStream_t s) {
  char *base = static_cast<char *>(ws);
  float *ws_l = reinterpret_cast<float *>(base + lay.e_off);
  int32_t *ws_count = reinterpret_cast<int32_t *>(base + lay.count_off);
  const size_t lds = std::max((size_t)lay.c_pad * sizeof(float) +
                                   (size_t)d.elig_words * sizeof(uint32_t) + (size_t)d.NB_max,
                               kScoreLdsBytes);
  forecast_select_kernel<<<dim3(lay.n_wg, d.P), kScoreThreads, lds, s>>>(
      d, st, f, ws_l, ws_count, lay.c_pad, lay.n_splits, lay.subs, sel, n_sel, kind, dbg);
  return hipGetLastError();
}

}  // namespace nosa
