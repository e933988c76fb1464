// C ABI entry points: argument checks (host only, before any HIP call),
// sizing, and launches. See include/nosa.h for the contract of each call.
#include <atomic>
#include <string>

#include "nosa_internal.h"

namespace {

std::atomic<int> g_tuning[NOSA_NUM_TUNE];

thread_local std::string g_last_error;

int fail(int code, const char *msg) {
  g_last_error = msg;
  return code;
}

int check_config(const nosa_config *c) {
  if (!c) return fail(NOSA_ERR_INVALID, "config is NULL");
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1)
    return fail(NOSA_ERR_INVALID, "batch and head counts must be positive");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(NOSA_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > nosa::kMaxGroup)
    return fail(NOSA_ERR_UNSUPPORTED, "query heads per KV head must be <= 16");
  if (c->head_dim != nosa::kHeadDim) return fail(NOSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (c->block_size != nosa::kBlock || c->pool_kernel != nosa::kPoolKernel ||
      c->pool_stride != nosa::kPoolStride)
    return fail(NOSA_ERR_UNSUPPORTED, "block/pool sizes must be 64/32/16");
  if (c->evict_hidden != 128) return fail(NOSA_ERR_UNSUPPORTED, "evict_hidden must be 128");
  if (c->n_sink_blocks < 0 || c->window_tokens < 0 || c->k_blocks < 0 ||
      c->k_q_blocks < 0 || c->k_e_blocks < 0)
    return fail(NOSA_ERR_INVALID, "negative budget or window");
  if (c->window_tokens % nosa::kBlock)
    return fail(NOSA_ERR_INVALID, "window_tokens must be a multiple of 64");
  if (c->window_tokens < 2 * nosa::kBlock)
    return fail(NOSA_ERR_UNSUPPORTED, "window_tokens must be >= 128");
  if (c->k_blocks != c->k_q_blocks + c->k_e_blocks)
    return fail(NOSA_ERR_INVALID, "k_blocks must equal k_q_blocks + k_e_blocks");
  if (c->k_e_blocks < c->n_sink_blocks + c->window_tokens / nosa::kBlock)
    return fail(NOSA_ERR_INVALID, "k_e_blocks must cover the sink and window blocks");
  if (c->k_blocks > nosa::kMaxK) return fail(NOSA_ERR_UNSUPPORTED, "k_blocks must be <= 128");
  if (c->max_context < nosa::kBlock || c->max_context > nosa::kMaxContext)
    return fail(NOSA_ERR_UNSUPPORTED, "max_context must be in [64, 262144]");
  if ((long)c->batch * c->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, "batch * n_kv_heads must be <= 65535");
  if (c->flags & ~(NOSA_EVICT_BIAS | NOSA_OFFLOAD)) return fail(NOSA_ERR_INVALID, "unknown flag bits");
  return NOSA_OK;
}

int make_dims(const nosa_config *c, nosa::Dims *d) {
  const int rc = check_config(c);
  if (rc) return rc;
  d->B = c->batch;
  d->Hq = c->n_q_heads;
  d->Hkv = c->n_kv_heads;
  d->G = c->n_q_heads / c->n_kv_heads;
  d->P = c->batch * c->n_kv_heads;
  d->max_context = c->max_context;
  d->NB_max = nosa::blocks_for(c->max_context);
  d->NB_kv = nosa::kv_blocks_per_pair(d->NB_max);
  d->tok_stride = d->NB_kv * nosa::kBlock;
  d->C_max = nosa::chunks_for(c->max_context);
  d->elig_words = (d->NB_max + 31) / 32;
  d->n_sink = c->n_sink_blocks;
  d->n_win = c->window_tokens / nosa::kBlock;
  d->k = c->k_blocks;
  d->k_q = c->k_q_blocks;
  d->k_e_dyn = c->k_e_blocks - c->n_sink_blocks - d->n_win;
  d->offload = (c->flags & NOSA_OFFLOAD) ? 1 : 0;
  d->bias = (c->flags & NOSA_EVICT_BIAS) ? 1 : 0;
  d->pool_small = nosa::tuning(NOSA_TUNE_SELECT_POOL) == 1 ? 0 : 1;
  return NOSA_OK;
}

int check_state(const nosa::Dims &d, const nosa_state *st) {
  if (!st) return fail(NOSA_ERR_INVALID, "state is NULL");
  if (!st->seq_len || !st->arrive || !st->status || !st->ckey || !st->tok_s ||
      !st->chunk_e || !st->blk_e || !st->eligible || !st->tail_keys || !st->kv_dev ||
      !st->w1 || !st->w2)
    return fail(NOSA_ERR_INVALID, "a state buffer is NULL");
  if (d.offload && (!st->kv_host || !st->slot_of_block || !st->block_of_slot))
    return fail(NOSA_ERR_INVALID, "offload mode needs kv_host and the slot maps");
  return NOSA_OK;
}

int check_len(const nosa::Dims &d, int32_t max_len_host) {
  if (max_len_host < 0 || max_len_host > d.max_context)
    return fail(NOSA_ERR_CAPACITY, "max_len_host outside [0, max_context]");
  return NOSA_OK;
}

int check_ws(const void *ws, size_t have, size_t need) {
  if (need && !ws) return fail(NOSA_ERR_WORKSPACE, "workspace is NULL");
  if (have < need) return fail(NOSA_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(NOSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return NOSA_OK;
}

int hip_result(hipError_t e) {
  if (e == hipSuccess) return NOSA_OK;
  g_last_error = std::string("HIP: ") + hipGetErrorString(e);
  return NOSA_ERR_HIP;
}

}  // namespace

int nosa::tuning(int knob) {
  return knob >= 0 && knob < NOSA_NUM_TUNE ? g_tuning[knob].load(std::memory_order_relaxed) : 0;
}

extern "C" {

int nosa_set_tuning(int knob, int32_t value) {
  bool ok = false;
  switch (knob) {
    case NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT: ok = value == 0 || (value >= 4 && value <= 64); break;
    case NOSA_TUNE_SELECT_SUBS: ok = value >= 0 && value <= 2048; break;
    case NOSA_TUNE_GATHER_VPT: ok = value == 0 || value == 1 || value == 2 || value == 4 || value == 8; break;
    case NOSA_TUNE_SELECT_POOL: ok = value >= 0 && value <= 2; break;
    default: break;
  }
  if (!ok) return fail(NOSA_ERR_INVALID, "unknown tuning knob or value out of range");
  return g_tuning[knob].exchange(value, std::memory_order_relaxed);
}

int nosa_hbm_read(const void *src, size_t bytes, int32_t n_workgroups, void *sink,
                  hipStream_t stream) {
  if (!src || !sink) return fail(NOSA_ERR_INVALID, "src / sink is NULL");
  if (bytes % 16) return fail(NOSA_ERR_INVALID, "bytes must be a multiple of 16");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15u)
    return fail(NOSA_ERR_INVALID, "src and sink must be 16-byte aligned");
  if (n_workgroups < 1 || n_workgroups > NOSA_MAX_READ_WORKGROUPS)
    return fail(NOSA_ERR_INVALID, "n_workgroups outside [1, NOSA_MAX_READ_WORKGROUPS]");
  return hip_result(nosa::launch_hbm_read(src, bytes, n_workgroups, sink, stream));
}

int nosa_link_copy(const void *src, void *dst, size_t bytes, int32_t n_workgroups,
                   hipStream_t stream) {
  if (!src || !dst) return fail(NOSA_ERR_INVALID, "src / dst is NULL");
  if (bytes % 16) return fail(NOSA_ERR_INVALID, "bytes must be a multiple of 16");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return fail(NOSA_ERR_INVALID, "src and dst must be 16-byte aligned");
  if (n_workgroups < 1 || n_workgroups > NOSA_MAX_FETCH_WORKGROUPS)
    return fail(NOSA_ERR_INVALID, "n_workgroups outside [1, NOSA_MAX_FETCH_WORKGROUPS]");
  if (bytes == 0) return NOSA_OK;
  return hip_result(nosa::launch_link_copy(src, dst, bytes, n_workgroups, stream));
}

int nosa_validate_config(const nosa_config *cfg) { return check_config(cfg); }

int nosa_state_bytes(const nosa_config *cfg, size_t out[NOSA_NUM_BUFFERS]) {
  nosa::Dims d;
  const int rc = make_dims(cfg, &d);
  if (rc) return rc;
  if (!out) return fail(NOSA_ERR_INVALID, "sizes_out is NULL");
  const size_t P = d.P, blk = (size_t)nosa::kBlockElems * 2;
  out[NOSA_BUF_SEQ_LEN] = (size_t)d.B * 4;
  out[NOSA_BUF_ARRIVE] = (size_t)d.B * 4;
  out[NOSA_BUF_STATUS] = 4;
  out[NOSA_BUF_CKEY] = P * d.C_max * nosa::kHeadDim * 2;
  out[NOSA_BUF_TOK_S] = P * d.tok_stride * 4;
  out[NOSA_BUF_CHUNK_E] = P * d.C_max * 4;
  out[NOSA_BUF_BLK_E] = P * d.NB_max * 4;
  out[NOSA_BUF_ELIGIBLE] = P * d.elig_words * 4;
  out[NOSA_BUF_TAIL_KEYS] = P * nosa::kPoolKernel * nosa::kHeadDim * 2;
  out[NOSA_BUF_KV_DEV] = P * (d.offload ? (size_t)d.k + 1 : (size_t)d.NB_kv) * blk;
  out[NOSA_BUF_KV_HOST] = d.offload ? P * d.NB_kv * blk : 0;
  out[NOSA_BUF_SLOT_OF_BLOCK] = d.offload ? P * d.NB_max * 4 : 0;
  out[NOSA_BUF_BLOCK_OF_SLOT] = d.offload ? P * (d.k + 1) * 4 : 0;
  out[NOSA_BUF_W1] = (size_t)d.Hkv * nosa::kHeadDim * nosa::kHeadDim * 2;
  out[NOSA_BUF_W2] = (size_t)d.Hkv * nosa::kHeadDim * 2;
  return NOSA_OK;
}

size_t nosa_workspace_bytes(const nosa_config *cfg, int which, int32_t max_len) {
  nosa::Dims d;
  if (make_dims(cfg, &d)) return 0;
  if (max_len < 0 || max_len > d.max_context) return 0;
  switch (which) {
    case NOSA_WS_SELECT: return nosa::select_layout(d, max_len).bytes;
    case NOSA_WS_FETCH: return nosa::fetch_layout(d).bytes;
    case NOSA_WS_DECODE: return nosa::decode_layout(d).bytes;
    default: return 0;
  }
}

int nosa_prefill_init(const nosa_config *cfg, const nosa_state *st, int32_t max_len_host,
                      hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  return hip_result(nosa::launch_prefill(d, *st, max_len_host, stream));
}

int nosa_compress_append(const nosa_config *cfg, const nosa_state *st, const uint16_t *k_new,
                         const uint16_t *v_new, int32_t max_len_host, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!k_new || !v_new) return fail(NOSA_ERR_INVALID, "k_new / v_new is NULL");
  return hip_result(nosa::launch_append(d, *st, k_new, v_new, stream));
}

int nosa_select(const nosa_config *cfg, const nosa_state *st, const uint16_t *q, int32_t *sel,
                int32_t *n_sel, uint8_t *kind, float *dbg_qscore, void *ws, size_t ws_bytes,
                int32_t max_len_host, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!q || !sel || !n_sel) return fail(NOSA_ERR_INVALID, "q / sel / n_sel is NULL");
  const nosa::SelectLayout lay = nosa::select_layout(d, max_len_host);
  rc = check_ws(ws, ws_bytes, lay.bytes);
  if (rc) return rc;
  return hip_result(nosa::launch_select(d, *st, q, sel, n_sel, kind, dbg_qscore, ws, lay, stream));
}

int nosa_append_select(const nosa_config *cfg, const nosa_state *st, const uint16_t *k_new,
                       const uint16_t *v_new, const uint16_t *q, int32_t *sel, int32_t *n_sel,
                       uint8_t *kind, float *dbg_qscore, void *ws, size_t ws_bytes,
                       int32_t max_len_host, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!k_new || !v_new) return fail(NOSA_ERR_INVALID, "k_new / v_new is NULL");
  if (!q || !sel || !n_sel) return fail(NOSA_ERR_INVALID, "q / sel / n_sel is NULL");
  const nosa::SelectLayout lay = nosa::select_layout(d, max_len_host);
  rc = check_ws(ws, ws_bytes, lay.bytes);
  if (rc) return rc;
  return hip_result(nosa::launch_append_select(d, *st, k_new, v_new, q, sel, n_sel, kind,
                                               dbg_qscore, ws, lay, stream));
}

int nosa_select_forecast(const nosa_config *cfg, const nosa_state *st, const uint16_t *f,
                         int32_t *sel, int32_t *n_sel, uint8_t *kind, float *dbg_fscore,
                         void *ws, size_t ws_bytes, int32_t max_len_host, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!f || !sel || !n_sel) return fail(NOSA_ERR_INVALID, "f / sel / n_sel is NULL");
  const nosa::SelectLayout lay = nosa::select_layout(d, max_len_host);
  rc = check_ws(ws, ws_bytes, lay.bytes);
  if (rc) return rc;
  return hip_result(
      nosa::launch_select_forecast(d, *st, f, sel, n_sel, kind, dbg_fscore, ws, lay, stream));
}

static int fetch_common(const nosa_config *cfg, const nosa_state *st, const int32_t *sel,
                        const int32_t *n_sel, int32_t *phys, int32_t *n_miss, int n_wg,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (rc) return rc;
  if (!sel || !n_sel || !phys || !n_miss)
    return fail(NOSA_ERR_INVALID, "sel / n_sel / phys / n_miss is NULL");
  const nosa::FetchLayout lay = nosa::fetch_layout(d);
  if (d.offload) {
    rc = check_ws(ws, ws_bytes, lay.bytes);
    if (rc) return rc;
  }
  return hip_result(nosa::launch_fetch(d, *st, sel, n_sel, phys, n_miss, ws, lay, stream, n_wg));
}

int nosa_fetch_delta(const nosa_config *cfg, const nosa_state *st, const int32_t *sel,
                     const int32_t *n_sel, int32_t *phys, int32_t *n_miss, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  return fetch_common(cfg, st, sel, n_sel, phys, n_miss, 0, ws, ws_bytes, stream);
}

int nosa_fetch_delta_wg(const nosa_config *cfg, const nosa_state *st, const int32_t *sel,
                        const int32_t *n_sel, int32_t *phys, int32_t *n_miss,
                        int32_t n_workgroups, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (n_workgroups < 1 || n_workgroups > NOSA_MAX_FETCH_WORKGROUPS)
    return fail(NOSA_ERR_INVALID, "n_workgroups outside [1, NOSA_MAX_FETCH_WORKGROUPS]");
  return fetch_common(cfg, st, sel, n_sel, phys, n_miss, n_workgroups, ws, ws_bytes, stream);
}

static int decode_common(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                         const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                         float *out, void *ws, size_t ws_bytes, int32_t max_len_host,
                         hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!q || !sel || !phys || !n_sel || !out)
    return fail(NOSA_ERR_INVALID, "q / sel / phys / n_sel / out is NULL");
  const nosa::DecodeLayout lay = nosa::decode_layout(d);
  rc = check_ws(ws, ws_bytes, lay.bytes);
  if (rc) return rc;
  return hip_result(nosa::launch_decode(d, *st, q, sel, phys, n_sel, out, ws, lay, stream,
                                        ev_start, ev_stop));
}

int nosa_sparse_decode(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                       const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                       float *out, void *ws, size_t ws_bytes, int32_t max_len_host,
                       hipStream_t stream) {
  return decode_common(cfg, st, q, sel, phys, n_sel, out, ws, ws_bytes, max_len_host, stream,
                       nullptr, nullptr);
}

int nosa_sparse_decode_timed(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                             const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                             float *out, void *ws, size_t ws_bytes, int32_t max_len_host,
                             hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event) {
  if (!start_event || !stop_event) return fail(NOSA_ERR_INVALID, "start / stop event is NULL");
  return decode_common(cfg, st, q, sel, phys, n_sel, out, ws, ws_bytes, max_len_host, stream,
                       start_event, stop_event);
}

int nosa_sparse_decode_static(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                              const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                              float *out, int32_t max_len_host, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (!rc) rc = check_len(d, max_len_host);
  if (rc) return rc;
  if (!q || !sel || !phys || !n_sel || !out)
    return fail(NOSA_ERR_INVALID, "q / sel / phys / n_sel / out is NULL");
  const nosa::DecodeLayout lay = nosa::decode_layout(d);
  if (lay.bytes > nosa::kDecodeStaticScratchBytes)
    return fail(NOSA_ERR_WORKSPACE,
                "decode workspace of this config exceeds NOSA_DECODE_STATIC_SCRATCH_BYTES; "
                "use nosa_sparse_decode with a caller workspace");
  return hip_result(nosa::launch_decode_static(d, *st, q, sel, phys, n_sel, out, lay, stream));
}

int nosa_prefill_block_scores(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                              int32_t n_queries, int32_t pos0, float *out, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (rc) return rc;
  if (!q || !out) return fail(NOSA_ERR_INVALID, "q / out is NULL");
  if (n_queries < 1 || pos0 < 0) return fail(NOSA_ERR_INVALID, "n_queries < 1 or pos0 < 0");
  if ((long)pos0 + n_queries > d.max_context)
    return fail(NOSA_ERR_CAPACITY, "pos0 + n_queries beyond max_context");
  return hip_result(nosa::launch_prefill_block_scores(d, *st, q, n_queries, pos0, out, stream));
}

int nosa_prefill_select(const nosa_config *cfg, const nosa_state *st, const float *scores,
                        int32_t n_queries, int32_t pos0, int32_t *sel, int32_t *n_sel,
                        hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (rc) return rc;
  if (!scores || !sel || !n_sel) return fail(NOSA_ERR_INVALID, "scores / sel / n_sel is NULL");
  if (n_queries < 1 || pos0 < 0) return fail(NOSA_ERR_INVALID, "n_queries < 1 or pos0 < 0");
  if ((long)pos0 + n_queries > d.max_context)
    return fail(NOSA_ERR_CAPACITY, "pos0 + n_queries beyond max_context");
  return hip_result(nosa::launch_prefill_select(d, *st, scores, n_queries, pos0, sel, n_sel, stream));
}

int nosa_prefill_attend(const nosa_config *cfg, const nosa_state *st, const uint16_t *q,
                        int32_t n_queries, int32_t pos0, const int32_t *sel,
                        const int32_t *n_sel, float *out, hipStream_t stream) {
  nosa::Dims d;
  int rc = make_dims(cfg, &d);
  if (!rc) rc = check_state(d, st);
  if (rc) return rc;
  if (d.offload) return fail(NOSA_ERR_UNSUPPORTED, "sparse prefill reads resident KV only");
  if (!q || !sel || !n_sel || !out) return fail(NOSA_ERR_INVALID, "q / sel / n_sel / out is NULL");
  if (n_queries < 1 || pos0 < 0) return fail(NOSA_ERR_INVALID, "n_queries < 1 or pos0 < 0");
  if ((long)pos0 + n_queries > d.max_context)
    return fail(NOSA_ERR_CAPACITY, "pos0 + n_queries beyond max_context");
  return hip_result(
      nosa::launch_prefill_attend(d, *st, q, n_queries, pos0, sel, n_sel, out, stream));
}

int nosa_host_alias(void *pinned_host_ptr, void **dev_alias) {
  if (!pinned_host_ptr || !dev_alias) return fail(NOSA_ERR_INVALID, "NULL argument");
  return hip_result(hipHostGetDevicePointer(dev_alias, pinned_host_ptr, 0));
}

const char *nosa_strerror(int code) {
  switch (code) {
    case NOSA_OK: return "ok";
    case NOSA_ERR_INVALID: return "invalid argument";
    case NOSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case NOSA_ERR_CAPACITY: return "length beyond max_context";
    case NOSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NOSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

const char *nosa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
