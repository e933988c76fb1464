// Host-side launchers and workspace layouts shared by the C ABI and the
// kernel files. Not part of the public ABI.
#pragma once

#include <stddef.h>

#include "nosa_common.h"

namespace nosa {

// Current value of a nosa_set_tuning knob (0: the library's choice).
int tuning(int knob);

// --- select workspace: per-pair chunk weights e = exp(l - m_split) for each
// head of the group, and per-(split, head) (m_split, Z_split).
constexpr int kChunksPerSplit = 128;   // 4 waves x one 32-chunk MFMA group

struct SelectLayout {
  int n_splits;      // chunk splits per pair
  int subs;          // splits scored by one workgroup, one after another
  int n_wg;          // scoring workgroups per pair: ceil(n_splits / subs)
  int c_pad;         // n_splits * kChunksPerSplit
  // count: per-pair arrivals, zero at rest, always at offset 0
  size_t count_off, e_off, stats_off, bytes;
};
SelectLayout select_layout(const Dims &d, int max_len);
size_t select_dyn_lds(const Dims &d, const SelectLayout &lay);   // pooling's dynamic LDS

// --- fetch workspace: per-pair copy list of (block, slot).
struct FetchLayout {
  size_t list_off, bytes;
};
FetchLayout fetch_layout(const Dims &d);

// --- decode workspace: split-K partials and one arrival counter per pair
// (zero at rest: the last workgroup of a pair resets it).
struct DecodeLayout {
  int blocks_per_split, n_splits;
  size_t count_off, o_off, ml_off, bytes;   // count at offset 0
};
DecodeLayout decode_layout(const Dims &d);

hipError_t launch_prefill(const Dims &d, const nosa_state &st, int max_len,
                          hipStream_t s);
hipError_t launch_append(const Dims &d, const nosa_state &st,
                         const uint16_t *k_new, const uint16_t *v_new,
                         hipStream_t s);
hipError_t launch_select(const Dims &d, const nosa_state &st,
                         const uint16_t *q, int32_t *sel, int32_t *n_sel,
                         uint8_t *kind, float *dbg_qscore, void *ws,
                         const SelectLayout &lay, hipStream_t s);
hipError_t launch_append_select(const Dims &d, const nosa_state &st,
                                const uint16_t *k_new, const uint16_t *v_new,
                                const uint16_t *q, int32_t *sel, int32_t *n_sel,
                                uint8_t *kind, float *dbg_qscore, void *ws,
                                const SelectLayout &lay, hipStream_t s);
hipError_t launch_select_forecast(const Dims &d, const nosa_state &st,
                                  const uint16_t *f, int32_t *sel,
                                  int32_t *n_sel, uint8_t *kind,
                                  float *dbg_fscore, void *ws,
                                  const SelectLayout &lay, hipStream_t s);
hipError_t launch_prefill_block_scores(const Dims &d, const nosa_state &st,
                                       const uint16_t *q, int T, int pos0,
                                       float *out, hipStream_t s);
hipError_t launch_prefill_select(const Dims &d, const nosa_state &st,
                                 const float *scores, int T, int pos0,
                                 int32_t *sel, int32_t *n_sel, hipStream_t s);
hipError_t launch_prefill_attend(const Dims &d, const nosa_state &st,
                                 const uint16_t *q, int T, int pos0,
                                 const int32_t *sel, const int32_t *n_sel,
                                 float *out, hipStream_t s);
hipError_t launch_hbm_read(const void *src, size_t bytes, int n_wg, void *sink,
                           hipStream_t s);
hipError_t launch_link_copy(const void *src, void *dst, size_t bytes, int n_wg,
                            hipStream_t s);
// n_wg > 0: copy with that many looping workgroups; 0: one per list entry
hipError_t launch_fetch(const Dims &d, const nosa_state &st,
                        const int32_t *sel, const int32_t *n_sel,
                        int32_t *phys, int32_t *n_miss, void *ws,
                        const FetchLayout &lay, hipStream_t s, int n_wg = 0);
// Size of the static scratch that nosa_sparse_decode_static uses in place of
// a caller's workspace.
constexpr size_t kDecodeStaticScratchBytes = size_t(8) << 20;
static_assert(kDecodeStaticScratchBytes == NOSA_DECODE_STATIC_SCRATCH_BYTES,
              "static scratch size differs from the header's");
hipError_t launch_decode_static(const Dims &d, const nosa_state &st, const uint16_t *q,
                                const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                                float *out, const DecodeLayout &lay, hipStream_t s);
// With ev_start / ev_stop, the launch records the kernel's own start and end
// into them (hipExtLaunchKernel).
hipError_t launch_decode(const Dims &d, const nosa_state &st,
                         const uint16_t *q, const int32_t *sel,
                         const int32_t *phys, const int32_t *n_sel,
                         float *out, void *ws, const DecodeLayout &lay,
                         hipStream_t s, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);

}  // namespace nosa
