// One launch for a decode step's append and selection (the two first steps
// of aiwiki "NOSA", How NOSA works, in order), for callers that run them
// back to back: the separate append launch and its dispatch disappear.
//
// grid (scoring workgroups + 1, pairs), 256 threads, a pair's workgroups on
// one XCD and each XCD's dispatched split by split (grid_unit_x_major):
//  - the last workgroup of a pair appends the token (K, V, ring, eviction
//    score, and the compressed key, chunk score and block score the token
//    completes);
//  - the others score their splits (one each unless NOSA_TUNE_SELECT_SUBS
//    asks for several) as the select
//    kernel does, in parallel, and arrive on the pair's counter; the last of
//    them pools and selects. The selection does not wait for the append:
//    the only thing it needs from it is the key of a chunk the token
//    completes, which the split holding that chunk builds itself from the
//    key ring and the new key (the same bits the append stores); the block
//    score the append may finalise belongs to a window block, which is
//    never a candidate;
//  - every pool and every append of a sequence arrive on the sequence's
//    counter once they have read its length (a pool as it starts pooling,
//    an append when done); the last of them advances it.
#include "nosa_append_dev.h"
#include "nosa_select_dev.h"

namespace nosa {
namespace {

template <bool MULTI>
__global__ __launch_bounds__(kScoreThreads, 4) void append_select_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const uint16_t *__restrict__ q, float *ws_e, float *ws_stats, int32_t *ws_count, int c_pad,
    int n_splits, int subs, int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
    uint8_t *__restrict__ kind_out, float *__restrict__ dbg) {
  int wg, p;
  grid_unit_x_major(wg, p);
  NOSA_PHASE(p, wg, 0);
  const int n_wg = gridDim.x - 1;
  const int b = p / d.Hkv, g = p % d.Hkv;
  // the append's LDS and the pooling's share the dynamic region (the append
  // workgroup never pools)
  extern __shared__ __align__(16) uint8_t dyn_sh[];
  AppendLds &ash = *reinterpret_cast<AppendLds *>(dyn_sh);
  __shared__ int sm_last;
  const int pos = st.seq_len[b];
  const bool ok = pos >= 0 && pos < d.max_context;
  const int L = ok ? pos + 1 : pos;
  // the last of the sequence's pools and appends to arrive on its counter
  // (each after reading the length) advances the length and leaves the
  // counter at zero
  auto advance = [&](int old) {
    if (old == 2 * d.Hkv - 1) {
      __hip_atomic_store(&st.arrive[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ok) __hip_atomic_store(&st.seq_len[b], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else atomicOr(st.status, NOSA_STATUS_CAPACITY);
    }
  };
  if (wg == n_wg) {                                       // uniform
    append_pair<kScoreThreads>(d, st, k_new, v_new, b, g, pos, true, ash);
    NOSA_PHASE(p, wg, 1);
    if (threadIdx.x == 0)
      advance(__hip_atomic_fetch_add(&st.arrive[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  } else {
    score_splits<MULTI>(d, st, q, L, ws_e, ws_stats, c_pad, n_splits, subs, wg, p,
                        ok ? k_new : nullptr);
    NOSA_PHASE(p, wg, 1);
    __builtin_amdgcn_s_waitcnt(0);          // this thread's stores have landed
    __syncthreads();
    NOSA_PHASE(p, wg, 2);
    if (threadIdx.x == 0)
      sm_last = __hip_atomic_fetch_add(&ws_count[p], 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == n_wg - 1;
    __syncthreads();
    NOSA_PHASE(p, wg, 3);
    if (!sm_last) return;
    // the pool arrives on the sequence's counter before pooling (it and its
    // scoring peers have read the length): the round trip runs under the
    // pooling instead of after its last step (issued behind the pooling's
    // first loads instead, it measured slower)
    int old = 0;
    if (threadIdx.x == 0)
      old = __hip_atomic_fetch_add(&st.arrive[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pool_select(d, st, L, ws_e, ws_stats, c_pad, n_splits, sel, n_sel, kind_out, dbg, p);
    if (threadIdx.x == 0) {
      __hip_atomic_store(&ws_count[p], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      advance(old);
    }
  }
  if (wg == n_wg) NOSA_PHASE(p, wg, 2);
  else NOSA_PHASE(p, kPhasePoolRow, 11);
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

#ifdef NOSA_PHASE_CLOCKS
NOSA_PHASE_READER(nosa_phase_clocks_append_select)
#endif
