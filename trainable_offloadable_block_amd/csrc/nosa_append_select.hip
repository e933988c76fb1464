// One launch for a decode step's append and selection (the two first steps
// of aiwiki "NOSA", How NOSA works, in order), for callers that run them
// back to back: the separate append launch and its dispatch disappear.
//
// grid (scoring workgroups + 1, pairs), 256 threads:
//  - the last workgroup of a pair appends the token (K, V, ring, eviction
//    score, and the compressed key, chunk score and block score the token
//    completes, the last two stored device-coherently);
//  - the others score their splits (one or several each) as the select
//    kernel does (every chunk but the newest, which the append may be
//    writing), in parallel;
//  - all arrive on the pair's counter; the last one scores the newest chunk,
//    pools and selects (block scores read device-coherently);
//  - the last pair of a sequence to finish advances the sequence's length:
//    by then every workgroup of the sequence has read it.
#include "nosa_append_dev.h"
#include "nosa_select_dev.h"

namespace nosa {
namespace {

template <bool MULTI>
__global__ __launch_bounds__(kScoreThreads) void append_select_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const uint16_t *__restrict__ q, float *ws_e, float *ws_stats, int32_t *ws_count, int c_pad,
    int n_splits, int subs, int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
    uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  int wg, p;
  grid_unit(wg, p);
  const int n_wg = gridDim.x - 1;
  const int b = p / d.Hkv, g = p % d.Hkv;
  // the append's LDS and the pooling's share the dynamic region: the append
  // workgroup pools (if it arrives last) only after its append is done
  extern __shared__ __align__(16) uint8_t dyn_sh[];
  AppendLds &ash = *reinterpret_cast<AppendLds *>(dyn_sh);
  __shared__ int sm_last;
  const int pos = st.seq_len[b];
  const bool ok = pos >= 0 && pos < d.max_context;
  const int L = ok ? pos + 1 : pos;
  if (wg == n_wg) {                                       // uniform
    append_pair<kScoreThreads>(d, st, k_new, v_new, b, g, pos, true, ash);
  } else {
    score_splits<MULTI>(d, st.ckey, q, L, ws_e, ws_stats, c_pad, n_splits, subs, wg, p);
  }
  __builtin_amdgcn_s_waitcnt(0);          // this thread's stores have landed
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(&ws_count[p], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              n_wg;                      // n_wg score workgroups + the append
  __syncthreads();
  if (!sm_last) return;
  pool_select(d, st, q, L, ws_e, ws_stats, c_pad, n_splits, sel, n_sel, kind_out, dbg, p);
  if (threadIdx.x == 0) {
    __hip_atomic_store(&ws_count[p], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every workgroup of this pair has read the length; the last pair of
    // the sequence advances it (and leaves the sequence's counter at zero)
    const int old = __hip_atomic_fetch_add(&st.arrive[b], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (old == d.Hkv - 1) {
      __hip_atomic_store(&st.arrive[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ok) __hip_atomic_store(&st.seq_len[b], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else atomicOr(st.status, NOSA_STATUS_CAPACITY);
    }
  }
}

}  // namespace

hipError_t launch_append_select(const Dims &d, const nosa_state &st, const uint16_t *k_new,
                                const uint16_t *v_new, const uint16_t *q, int32_t *sel,
                                int32_t *n_sel, uint8_t *kind, float *dbg, void *ws,
                                const SelectLayout &lay, hipStream_t s) {
  char *base = static_cast<char *>(ws);
  float *ws_e = reinterpret_cast<float *>(base + lay.e_off);
  float *ws_stats = reinterpret_cast<float *>(base + lay.stats_off);
  int32_t *ws_count = reinterpret_cast<int32_t *>(base + lay.count_off);
  auto kernel = lay.subs > 1 ? append_select_kernel<true> : append_select_kernel<false>;
  const size_t lds = std::max(select_dyn_lds(d, lay), sizeof(AppendLds));
  kernel<<<dim3(lay.n_wg + 1, d.P), kScoreThreads, lds, s>>>(
      d, st, k_new, v_new, q, ws_e, ws_stats, ws_count, lay.c_pad, lay.n_splits, lay.subs, sel,
      n_sel, kind, dbg);
  return hipGetLastError();
}

}  // namespace nosa
