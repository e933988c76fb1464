// Two-stage block selection (aiwiki "NOSA", How NOSA works; NOSA-1B
// 核心组件揭秘, 核心组件三; l189 article, 2.1).
//
// select_kernel (chunk splits x pairs), one launch:
//  - every workgroup scores one split (several one after another when
//    NOSA_TUNE_SELECT_SUBS asks for it): query-aware logits of the GQA group against the
//    compressed keys on MFMA, l = q . c / sqrt(128) (kept in the log2 domain
//    for the hardware exp2); per split and head, m = max l (published in
//    the log2 domain), Z = sum exp(l - m); it publishes e = exp(l - m) per
//    chunk and (m, Z) with device-coherent stores and arrives on the pair's
//    counter; the newest chunk is left to
//  - the pair's last workgroup, which scores it, combines the split
//    statistics into the per-head softmax, sums the group's heads, max-pools
//    the chunks
//    overlapping each block, then stage 1 (top k_q by the query-aware score)
//    and stage 2 (top k_e' eligible by the agnostic score), each an exact
//    workgroup top-k by histogram range refinement, writes the ascending
//    selection and clears the eligibility of every candidate left out (never
//    re-selected by the agnostic stage).
#include <algorithm>

#include "nosa_select_dev.h"

namespace nosa {
namespace {

// grid (scoring workgroups, pairs): every workgroup scores its `subs`
// splits and arrives on the pair's counter once its results have landed; the
// last one pools and selects, then resets the counter (zero at rest).
template <bool MULTI>
__global__ __launch_bounds__(kScoreThreads, 4) void select_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ q, float *ws_e, float *ws_stats,
    int32_t *ws_count, int c_pad, int n_splits, int subs, int32_t *__restrict__ sel,
    int32_t *__restrict__ n_sel, uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  int wg, p;
  grid_unit_x_major(wg, p);
  __shared__ int sm_last;
  const int L = st.seq_len[p / d.Hkv];
  score_splits<MULTI>(d, st, q, L, ws_e, ws_stats, c_pad, n_splits, subs, wg, p);
  __builtin_amdgcn_s_waitcnt(0);          // this thread's stores have landed
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(&ws_count[p], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (int)gridDim.x - 1;
  __syncthreads();
  if (!sm_last) return;
  pool_select(d, st, L, ws_e, ws_stats, c_pad, n_splits, sel, n_sel, kind_out, dbg, p);
  if (threadIdx.x == 0) __hip_atomic_store(&ws_count[p], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

SelectLayout select_layout(const Dims &d, int max_len) {
  SelectLayout s;
  const int C = chunks_for(max_len);
  s.n_splits = C > 0 ? (C + kChunksPerSplit - 1) / kChunksPerSplit : 1;
  s.c_pad = s.n_splits * kChunksPerSplit;
  // one split per workgroup, however many rounds of workgroups that takes:
  // scoring several splits one after another in one round (the grid kept
  // to the chip's 4 resident workgroups per CU) measured slower on every
  // workload that needs it (offloaded 32K stack 377.3 against 373.8 K
  // tokens/s per layer with 3 splits per workgroup; 8B-shaped 64K layer
  // 89.6 against 87.8 K with 11)
  s.subs = 1;
  if (const int v = tuning(NOSA_TUNE_SELECT_SUBS)) s.subs = min(v, s.n_splits);
  s.n_wg = (s.n_splits + s.subs - 1) / s.subs;
  s.count_off = 0;
  s.e_off = (((size_t)d.P * sizeof(int32_t) + 255) & ~(size_t)255);
  s.stats_off = s.e_off +
                (((size_t)d.P * s.c_pad * padded_group(d.G) * sizeof(float) + 255) & ~(size_t)255);
  s.bytes = s.stats_off + (((size_t)d.P * s.n_splits * d.G * sizeof(float2) + 255) & ~(size_t)255);
  return s;
}

size_t select_dyn_lds(const Dims &d, const SelectLayout &lay) {
  // the pool's arrays, or the scoring waves' transpose space if larger (a
  // workgroup pools only after its scoring is done)
  return std::max(((size_t)lay.n_splits * padded_group(d.G) + lay.c_pad) * sizeof(float) +
                      (size_t)d.elig_words * sizeof(uint32_t) + (size_t)d.NB_max,
                  kScoreLdsBytes);
}

hipError_t launch_select(const Dims &d, const nosa_state &st, const uint16_t *q,
                         int32_t *sel, int32_t *n_sel, uint8_t *kind, float *dbg,
                         void *ws, const SelectLayout &lay, hipStream_t s) {
  char *base = static_cast<char *>(ws);
  float *ws_e = reinterpret_cast<float *>(base + lay.e_off);
  float *ws_stats = reinterpret_cast<float *>(base + lay.stats_off);
  int32_t *ws_count = reinterpret_cast<int32_t *>(base + lay.count_off);
  auto kernel = lay.subs > 1 ? select_kernel<true> : select_kernel<false>;
  kernel<<<dim3(lay.n_wg, d.P), kScoreThreads, select_dyn_lds(d, lay), s>>>(
      d, st, q, ws_e, ws_stats, ws_count, lay.c_pad, lay.n_splits, lay.subs, sel, n_sel, kind,
      dbg);
  return hipGetLastError();
}

}  // namespace nosa
