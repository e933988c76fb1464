/*
 * nosa.h -- C ABI of the NOSA batched decode-step hot path on MI355X (gfx950).
 *
 * NOSA (Native and Offloadable Sparse Attention) attends, at each decode
 * step, to an attention-sink block, a sliding window and k_q + k_e' dynamic
 * 64-token blocks, and keeps the full KV cache in pinned host memory with a
 * per-layer GPU cache of the previous step's blocks (aiwiki "NOSA", How NOSA
 * works and NOSI: the inference system; SparDA article on aliyun,
 * KV 预取的运行时实现). One decode step of one layer is four calls, in order:
 *
 *   nosa_compress_append  append the step's K, V; per-token eviction score;
 *                         CompressK chunk and block-score bookkeeping
 *   nosa_select           query-aware chunk scores, two-stage block selection
 *                         under the never-reselect rule
 *   nosa_fetch_delta      (offload only) set difference against the cached
 *                         blocks, then copy only the missing blocks from host
 *   nosa_sparse_decode    attention over the selected blocks with the
 *                         eviction-score logit bias
 *
 * SparDA's layer-ahead order (aliyun article on SparDA, 解耦选块与注意力计算
 * and KV 预取的运行时实现; aiwiki "NOSA", Adoption in SparDA) replaces the
 * first two calls: while layer l runs, nosa_select_forecast picks layer
 * l+1's blocks from a forecast head and nosa_fetch_delta_wg brings them in
 * on a second stream with a bounded number of workgroups; layer l+1 then
 * runs nosa_compress_append and nosa_sparse_decode.
 *
 * Conventions
 *  - Every pointer is caller-owned. The library never allocates or frees
 *    memory and keeps no device state of its own.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Calls only enqueue work on `stream` and return; none synchronises the
 *    host. One state is used from one stream at a time; distinct states are
 *    independent.
 *  - Argument checks are pure host code and run before any HIP call, so a
 *    rejected call enqueues nothing. Kernel launch failures return
 *    NOSA_ERR_HIP; nosa_last_error() then holds a message (thread-local).
 *    Conditions only the device can see (a sequence that would outgrow
 *    max_context) set bits in state->status and leave that sequence's data
 *    untouched; they surface when the caller reads status.
 *  - A pair is (sequence b, KV head g); pair index p = b * n_kv_heads + g.
 *    Query head h belongs to KV head h / (n_q_heads / n_kv_heads).
 *  - Launch shapes are chosen from the config and the length bound; tests
 *    and tuning sweeps can override three of them with nosa_set_tuning
 *    (results do not depend on them).
 */
#ifndef NOSA_H
#define NOSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ error codes */
enum {
  NOSA_OK = 0,
  NOSA_ERR_INVALID = -1,     /* NULL pointer, inconsistent budget or sizes  */
  NOSA_ERR_UNSUPPORTED = -2, /* a shape or parameter this build does not do */
  NOSA_ERR_CAPACITY = -3,    /* max_len_host beyond max_context             */
  NOSA_ERR_WORKSPACE = -4,   /* workspace missing or too small              */
  NOSA_ERR_HIP = -5          /* a HIP launch or runtime call failed         */
};

/* status bits written by kernels into state->status[0] */
#define NOSA_STATUS_CAPACITY 1u   /* an append found seq_len == max_context  */
#define NOSA_STATUS_BAD_SEL  2u   /* fetch/decode saw a block id out of range */
#define NOSA_STATUS_LEN_HINT 4u   /* select met a length above max_len_host   */
#define NOSA_STATUS_SHORT_CONTEXT 8u /* prefill scores asked past seq_len   */

/* largest workgroup budget nosa_fetch_delta_wg accepts */
#define NOSA_MAX_FETCH_WORKGROUPS 4096

/* config flags */
#define NOSA_EVICT_BIAS 1u /* add the eviction score s_j to the logits      */
#define NOSA_OFFLOAD    2u /* full KV lives in pinned host memory           */

/* ------------------------------------------------------------ config
 * Supported: head_dim 128; n_q_heads a multiple of n_kv_heads with group
 * size 1..16; block_size 64, pool_kernel 32, pool_stride 16 (aiwiki "NOSA",
 * Main-experiment configuration; NOSA-1B 核心组件揭秘, 核心组件一);
 * window_tokens a multiple of 64 and >= 128 (so every candidate block's
 * chunks are complete); k_blocks = k_q_blocks + k_e_blocks <= 128 with
 * k_e_blocks >= n_sink_blocks + window_tokens / 64 (k_e counts the sink and
 * window blocks, aiwiki "NOSA" Main-experiment configuration);
 * evict_hidden 128; 64 <= max_context <= 262144; batch * n_kv_heads <= 65535.
 */
typedef struct nosa_config {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t block_size, pool_kernel, pool_stride;
  int32_t n_sink_blocks, window_tokens;
  int32_t k_blocks, k_q_blocks, k_e_blocks;
  int32_t max_context, evict_hidden;
  uint32_t flags;
} nosa_config;

/* ------------------------------------------------------------ state
 * One layer's decode state. Sizes (in elements) come from nosa_state_bytes;
 * write C_max = (max_context - 32) / 16 + 1 chunks, NB_max =
 * ceil(max_context / 64) blocks, P = batch * n_kv_heads pairs, and NB_kv
 * = NB_max, or NB_max + 1 when NB_max is a multiple of 129, for the
 * per-pair stride of the KV pool, the host store and the token scores (a
 * stride of 258 blocks put the decode's reads of many pairs on a part of
 * the HBM channels: 13 % slower on MI355X; the extra block is never used).
 *
 * KV block layout (device pool, device cache and host store alike): one
 * block of one pair is 32 KiB = K then V, bf16:
 *     K part  [64 tokens][128 dims]   (row = token)
 *     V part  1 KiB tiles [2 halves][8 dim tiles][4 token groups][16 dims]
 *             [8 tokens]: token t, dim c at element
 *             ((((t/32)*8 + c/16)*4 + (t%32)/8)*16 + c%16)*8 + t%8
 *             (a tile is 16 dims x 32 tokens, one MFMA operand per wave)
 * A block is the pages' 16 KiB-per-tensor transfer unit (aiwiki "NOSA",
 * Main-experiment configuration), with K and V adjacent. Inside a
 * sequence's newest block the positions at and past seq_len hold zeros:
 * nosa_prefill_init clears them and nosa_compress_append clears a block when
 * a token opens it; callers must not write there between calls.
 */
typedef struct nosa_state {
  int32_t *seq_len;       /* dev [B]: tokens per sequence; +1 per append    */
  int32_t *arrive;        /* dev [B]: zero; append's per-sequence counter   */
  uint32_t *status;       /* dev [1]: NOSA_STATUS_* bits (sticky)           */
  uint16_t *ckey;         /* dev [P][C_max][128] bf16 compressed keys       */
  float *tok_s;           /* dev [P][NB_kv*64] eviction score per token     */
  float *chunk_e;         /* dev [P][C_max] mean eviction score per chunk   */
  float *blk_e;           /* dev [P][NB_max] query-agnostic block score     */
  uint32_t *eligible;     /* dev [P][ceil(NB_max/32)] never-reselect bits   */
  uint16_t *tail_keys;    /* dev [P][32][128] last 32 keys (ring by pos%32) */
  uint16_t *kv_dev;       /* dev: resident pool [P][NB_kv][32 KiB block] or
                             offload cache [P][k_blocks+1][32 KiB block]    */
  uint16_t *kv_host;      /* device-usable alias of the pinned host store
                             [P][NB_kv][32 KiB block]; NULL when resident   */
  int32_t *slot_of_block; /* dev [P][NB_max] cache slot or -1 (offload)     */
  int32_t *block_of_slot; /* dev [P][k_blocks+1] block id or -1 (offload)   */
  const uint16_t *w1;     /* dev [Hkv][128 in][128 hidden] bf16 eviction W1 */
  const uint16_t *w2;     /* dev [Hkv][128 hidden] bf16 eviction W2         */
} nosa_state;

enum {
  NOSA_BUF_SEQ_LEN = 0, NOSA_BUF_ARRIVE, NOSA_BUF_STATUS, NOSA_BUF_CKEY,
  NOSA_BUF_TOK_S, NOSA_BUF_CHUNK_E, NOSA_BUF_BLK_E, NOSA_BUF_ELIGIBLE,
  NOSA_BUF_TAIL_KEYS, NOSA_BUF_KV_DEV, NOSA_BUF_KV_HOST,
  NOSA_BUF_SLOT_OF_BLOCK, NOSA_BUF_BLOCK_OF_SLOT, NOSA_BUF_W1, NOSA_BUF_W2,
  NOSA_NUM_BUFFERS
};

/* kind codes written by nosa_select */
enum { NOSA_KIND_NONE = 0, NOSA_KIND_SINK = 1, NOSA_KIND_WINDOW = 2,
       NOSA_KIND_QUERY = 3, NOSA_KIND_AGNOSTIC = 4 };

/* workspace users */
enum { NOSA_WS_SELECT = 1, NOSA_WS_FETCH = 2, NOSA_WS_DECODE = 3 };

/* ------------------------------------------------------------ sizing */

/* Checks a config against the supported set. NOSA_OK, NOSA_ERR_INVALID or
 * NOSA_ERR_UNSUPPORTED. Host only. */
int nosa_validate_config(const nosa_config *cfg);

/* Byte size of every state buffer, indexed by NOSA_BUF_*. Buffers a mode
 * does not use (kv_host and the slot maps when resident) get 0. Host only. */
int nosa_state_bytes(const nosa_config *cfg, size_t sizes_out[NOSA_NUM_BUFFERS]);

/* Workspace bytes that call `which` needs for sequences up to max_len
 * tokens; 0 for an invalid config. A workspace must be 256-byte aligned.
 * The select and decode workspaces must be zero-filled before their first
 * use (each holds per-pair arrival counters that every call leaves at zero);
 * the fetch workspace needs no initialisation. */
size_t nosa_workspace_bytes(const nosa_config *cfg, int which, int32_t max_len);

/* ------------------------------------------------------------ calls */

/* Builds the decode state from a prefilled context (untimed set-up).
 * Precondition: seq_len[b] holds each sequence's prefilled length
 * (<= max_len_host <= max_context) and the context's K, V sit in kv_dev
 * (resident) or in the host store (offload) in the block layout above.
 * Computes tok_s for every token (eviction head, aiwiki "NOSA" How NOSA
 * works), every complete compressed key and chunk mean, blk_e of every
 * complete block, fills tail_keys, sets every eligible bit (E(0) = all
 * candidates), empties the offload cache, clears arrive and status. */
int nosa_prefill_init(const nosa_config *cfg, const nosa_state *st,
                      int32_t max_len_host, hipStream_t stream);

/* Appends one token per pair at position seq_len[b] and increments
 * seq_len[b]. k_new, v_new: dev bf16 [B][Hkv][128].
 *  - writes K, V into kv_dev (resident), or (offload) into the cache slot
 *    of its block, a token that opens a new block taking a free slot for it;
 *    the host store receives a block from its cache slot, whole, when the
 *    block's last token arrives (it stays cached until then: every
 *    selection holds the window), and a token whose block is not cached
 *    (before the first fetch) goes to the host store directly. A selection
 *    passed to nosa_fetch_delta must therefore include each sequence's
 *    newest block, as every nosa_select / nosa_select_forecast result does;
 *  - tok_s[pos] = softplus(v W1) W2 in fp32 (aiwiki "NOSA", How NOSA works;
 *    l189 article, 2.1, eq. 4);
 *  - when a 32-token chunk completes (L >= 32 and (L - 32) % 16 == 0):
 *    ckey = bf16 round-to-nearest-even of the exact mean of its 32 keys
 *    (NOSA-1B 核心组件揭秘, 核心组件一), chunk_e = mean of its tok_s, and
 *    when chunk 4b+3 completes, blk_e[b] = max of chunk_e over the chunks
 *    overlapping block b (l189 article, 2.1, eqs. 5-6).
 * max_len_host: an upper bound on seq_len after the call. */
int nosa_compress_append(const nosa_config *cfg, const nosa_state *st,
                         const uint16_t *k_new, const uint16_t *v_new,
                         int32_t max_len_host, hipStream_t stream);

/* Two-stage block selection for the current length L = seq_len[b].
 * q: dev bf16 [B][Hq][128] (post-RoPE query of the step).
 *  - query-aware score: per query head, softmax over all complete chunks of
 *    q . ckey / sqrt(128); summed over the GQA group; max-pooled over the
 *    chunks overlapping each block (NOSA-1B 核心组件揭秘, 核心组件三);
 *  - candidates: complete blocks in [n_sink, nb - n_win), nb = ceil(L/64);
 *  - stage 1: the k_q candidates of highest query-aware score; stage 2: the
 *    k_e - n_sink - n_win eligible remaining candidates of highest blk_e
 *    (aiwiki "NOSA", How NOSA works); ties go to the lower block id;
 *  - eligibility: a candidate not selected loses its bit for good.
 * Outputs: sel dev int32 [B][Hkv][k_blocks], the selected block ids in
 * ascending order, -1 padded; n_sel dev int32 [B][Hkv]; kind (optional) dev
 * uint8 [B][Hkv][k_blocks] NOSA_KIND_*; dbg_qscore (optional) dev fp32
 * [B][Hkv][NB_max], the query-aware block score of each candidate (other
 * entries untouched). ws: NOSA_WS_SELECT bytes, zero-filled before the
 * first call and left at zero by every call; calls that share one ws must be
 * ordered (one stream). */
int nosa_select(const nosa_config *cfg, const nosa_state *st,
                const uint16_t *q, int32_t *sel, int32_t *n_sel,
                uint8_t *kind, float *dbg_qscore, void *ws, size_t ws_bytes,
                int32_t max_len_host, hipStream_t stream);

/* nosa_compress_append followed by nosa_select, in one launch: the same
 * results (state, sel, n_sel, kind, dbg_qscore) as the two calls in a row
 * with the same arguments, the append's token at position seq_len[b] and
 * the selection at the new length. ws and max_len_host as for nosa_select
 * (max_len_host bounds the length after the append). For callers that run
 * the two steps back to back (one launch and its dispatch fewer). */
int nosa_append_select(const nosa_config *cfg, const nosa_state *st,
                       const uint16_t *k_new, const uint16_t *v_new,
                       const uint16_t *q, int32_t *sel, int32_t *n_sel,
                       uint8_t *kind, float *dbg_qscore, void *ws,
                       size_t ws_bytes, int32_t max_len_host,
                       hipStream_t stream);

/* SparDA's layer-ahead selection (aliyun article, 解耦选块与注意力计算 and
 * 轻量化设计与训练): the same two stages, eligibility rule and outputs as
 * nosa_select, taken BEFORE the step's token is appended, for the length
 * L = seq_len[b] + 1 that the next nosa_compress_append gives the sequence,
 * with stage 1 ranked by a forecast head instead of the group's queries:
 *  - f: dev bf16 [B][Hkv][128], one forecast head per KV group (produced by
 *    the previous layer);
 *  - forecast score of a block: max over the compressed keys overlapping it
 *    of f . ckey / sqrt(128), with no softmax and no sum over heads;
 *  - every candidate block's chunks exist before the append (window_tokens
 *    >= 128), so the coming token changes nothing but the window.
 * dbg_fscore (optional) dev fp32 [B][Hkv][NB_max]: the forecast score of
 * each candidate. ws: NOSA_WS_SELECT bytes, as for nosa_select;
 * max_len_host bounds seq_len + 1. The caller then runs nosa_fetch_delta
 * (or nosa_fetch_delta_wg), nosa_compress_append and nosa_sparse_decode on
 * this selection, with no other select call in between. */
int nosa_select_forecast(const nosa_config *cfg, const nosa_state *st,
                         const uint16_t *f, int32_t *sel, int32_t *n_sel,
                         uint8_t *kind, float *dbg_fscore, void *ws,
                         size_t ws_bytes, int32_t max_len_host,
                         hipStream_t stream);

/* Offload mode only: brings the selected blocks into the device cache.
 * Set difference of sel against the cached blocks (NOSI's set-difference
 * kernel, aiwiki "NOSA", NOSI: the inference system): slots whose block is
 * not selected are freed, each missing block gets a free slot and is copied
 * as one 32 KiB block from the host store (block-wise, not token-wise
 * transfers, aiwiki "NOSA", How NOSA works). A missing block that holds no
 * token yet (first position >= seq_len[b]: the block the next append opens,
 * which a layer-ahead selection includes) gets its slot but is not copied;
 * the append clears and fills it. Outputs: phys dev int32
 * [B][Hkv][k_blocks] = cache slot of each sel entry (-1 padded); n_miss dev
 * int32 [B][Hkv] = blocks copied. ws: NOSA_WS_FETCH bytes. */
int nosa_fetch_delta(const nosa_config *cfg, const nosa_state *st,
                     const int32_t *sel, const int32_t *n_sel, int32_t *phys,
                     int32_t *n_miss, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* nosa_fetch_delta with the copies made by n_workgroups workgroups that
 * loop over the missing blocks (1 <= n_workgroups <=
 * NOSA_MAX_FETCH_WORKGROUPS), SparDA's persistent copy kernel with a
 * workgroup budget (aliyun article, KV 预取的运行时实现): for a fetch that
 * runs beside compute on another stream and should hold only that many
 * workgroup slots. Same outputs, state changes and ws as nosa_fetch_delta;
 * in resident mode identical to it. */
int nosa_fetch_delta_wg(const nosa_config *cfg, const nosa_state *st,
                        const int32_t *sel, const int32_t *n_sel,
                        int32_t *phys, int32_t *n_miss, int32_t n_workgroups,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* Sparse attention for the step. For query head h of pair (b, g):
 *   out[b][h] = sum_j softmax_j(q_h . k_j / sqrt(128) + beta * tok_s[j]) v_j
 * over the existing tokens (j < seq_len[b]) of the blocks listed in sel;
 * beta = 1 with NOSA_EVICT_BIAS, else 0 (aiwiki "NOSA", How NOSA works;
 * l189 article, 2.1, eq. 8). K, V are read from kv_dev at block index
 * phys[i] (resident: pass phys = sel). out: dev fp32 [B][Hq][128].
 * ws: NOSA_WS_DECODE bytes, zero-filled before its first use. */
int nosa_sparse_decode(const nosa_config *cfg, const nosa_state *st,
                       const uint16_t *q, const int32_t *sel,
                       const int32_t *phys, const int32_t *n_sel, float *out,
                       void *ws, size_t ws_bytes, int32_t max_len_host,
                       hipStream_t stream);

/* nosa_sparse_decode whose kernel launch also stamps its own start and end
 * into start_event and stop_event (hipExtLaunchKernel): the interval the
 * command processor records for the dispatch, as a kernel trace reports it,
 * without the dispatch gap that a hipEventRecord pair around the call adds.
 * Both events are caller-created (hipEventCreate, timing enabled) and
 * caller-owned; NULL for either returns NOSA_ERR_INVALID. Same outputs,
 * state changes and ws as nosa_sparse_decode. */
int nosa_sparse_decode_timed(const nosa_config *cfg, const nosa_state *st,
                             const uint16_t *q, const int32_t *sel,
                             const int32_t *phys, const int32_t *n_sel,
                             float *out, void *ws, size_t ws_bytes,
                             int32_t max_len_host, hipStream_t stream,
                             hipEvent_t start_event, hipEvent_t stop_event);

/* Size of the scratch that nosa_sparse_decode_static uses (8 MiB). */
#define NOSA_DECODE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)

/* nosa_sparse_decode for callers that cannot allocate memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same kernels, results and state changes (bit for bit), with the
 * decode workspace taken from a scratch array built into the library
 * instead of a caller's ws. No call allocates or frees anything.
 *  - Each GPU holds its own NOSA_DECODE_STATIC_SCRATCH_BYTES copy of the
 *    scratch until the process ends; its address is looked up on the first
 *    call on that device (with that device current).
 *  - A config whose decode workspace (nosa_workspace_bytes(cfg,
 *    NOSA_WS_DECODE, ...)) exceeds NOSA_DECODE_STATIC_SCRATCH_BYTES returns
 *    NOSA_ERR_WORKSPACE and enqueues nothing.
 *  - Every call on a GPU shares that GPU's scratch, which keeps the last
 *    call's contents; calls that overlap on one GPU (different streams, or
 *    a graph replay beside an eager call) race and must be ordered by the
 *    caller. A call whose per-pair arrival counters reach past the previous
 *    call's first clears them with a small fill kernel on `stream` (no
 *    memset node), so a call's counters always start at zero. */
int nosa_sparse_decode_static(const nosa_config *cfg, const nosa_state *st,
                              const uint16_t *q, const int32_t *sel,
                              const int32_t *phys, const int32_t *n_sel,
                              float *out, int32_t max_len_host,
                              hipStream_t stream);

/* Block scores of many prompt queries at once: the selection side of NOSA_S's
 * sparse prefill (aiwiki "NOSA", Results: NOSA_S is sparse in both phases),
 * each query scored exactly as a decode step at its own length would score it
 * (the query-aware score of nosa_select; NOSA-1B 核心组件揭秘, 核心组件三).
 * q: dev bf16 [B][n_queries][Hq][128]; query i of every sequence sits at
 * position pos0 + i, and the state (nosa_prefill_init) must already hold the
 * prompt up to pos0 + n_queries (seq_len[b] >= pos0 + n_queries; a sequence
 * that falls short sets NOSA_STATUS_SHORT_CONTEXT and gets no output).
 * out: dev fp32 [B][Hkv][n_queries][nb], nb = ceil((pos0 + n_queries) / 64):
 * row i holds, for each candidate block of length L = pos0 + i + 1 (between
 * the sink and L's window), the max over the block's chunks of the sum over
 * the group's heads of the per-head softmax over the chunks complete at L of
 * q . ckey / sqrt(128); -inf for every other block. One dense MFMA product
 * per (query, head) row against the compressed keys. */
int nosa_prefill_block_scores(const nosa_config *cfg, const nosa_state *st,
                              const uint16_t *q, int32_t n_queries,
                              int32_t pos0, float *out, hipStream_t stream);

/* Sparse prefill selection, NOSA_S style (aiwiki "NOSA", Results; aiwiki
 * "NOSA", How NOSA works): for each of n_queries prompt queries (query i at
 * position pos0 + i, length L = pos0 + i + 1), NOSA's two stages with every
 * candidate eligible (the never-reselect state begins with decoding): the
 * k_q candidates of highest block score, then the k_e - n_sink - n_win
 * others of highest blk_e; ties to the lower block id. scores: the output of
 * nosa_prefill_block_scores for the same n_queries and pos0. Outputs: sel
 * dev int32 [B][Hkv][n_queries][k_blocks], each row the ascending list of
 * sink, window and selected blocks, -1 padded; n_sel dev int32
 * [B][Hkv][n_queries]. */
int nosa_prefill_select(const nosa_config *cfg, const nosa_state *st,
                        const float *scores, int32_t n_queries, int32_t pos0,
                        int32_t *sel, int32_t *n_sel, hipStream_t stream);

/* Sparse prefill attention (resident KV only): each prompt query attends as
 * a decode step at its own length would (nosa_sparse_decode's formula), over
 * the tokens at or before its position in the blocks of its row of sel.
 * q: dev bf16 [B][n_queries][Hq][128]; sel, n_sel from nosa_prefill_select
 * with the same n_queries and pos0; out: dev fp32 [B][n_queries][Hq][128].
 * An entry that names a block past the query's position or beyond NB_max is
 * skipped and sets NOSA_STATUS_BAD_SEL. Offload configs get
 * NOSA_ERR_UNSUPPORTED. */
int nosa_prefill_attend(const nosa_config *cfg, const nosa_state *st,
                        const uint16_t *q, int32_t n_queries, int32_t pos0,
                        const int32_t *sel, const int32_t *n_sel, float *out,
                        hipStream_t stream);

/* Device-usable address of pinned host memory (hipHostGetDevicePointer);
 * allocates nothing. */
int nosa_host_alias(void *pinned_host_ptr, void **dev_alias);

/* Copies `bytes` (a multiple of 16) from src to dst with n_workgroups
 * workgroups of 256 threads reading 16 bytes per thread and load, the load
 * path of nosa_fetch_delta's copies. src may be a device-usable alias of
 * pinned host memory (nosa_host_alias): the host-link ceiling that a delta
 * fetch is measured against (aiwiki "NOSA", NOSI: the inference system: the
 * GPU kernel that reads host memory directly, against the link's peak).
 * 1 <= n_workgroups <= NOSA_MAX_FETCH_WORKGROUPS. */
int nosa_link_copy(const void *src, void *dst, size_t bytes, int32_t n_workgroups,
                   hipStream_t stream);

/* Reads `bytes` (a multiple of 16) of device memory at src with n_workgroups
 * workgroups of 256 threads, each over its own contiguous span (the bytes
 * split evenly, the last spans shorter or empty), with non-temporal 16-byte loads, 8
 * in flight per thread, and writes each thread's XOR of what it read as one
 * 16-byte word to sink[workgroup * 256 + thread] (the caller's n_workgroups * 4 KiB
 * of device memory; the XOR of all of them is the XOR of the buffer). The
 * HBM read rate of a kernel that does nothing else: the practical ceiling
 * beside the published peak that the decode's streaming (NOSA-1B 核心组件揭秘,
 * 解码阶段如何只用 64 个 KV 块: the selected blocks' K and V read once per
 * step) is reported against. src and sink 16-byte aligned;
 * 1 <= n_workgroups <= NOSA_MAX_READ_WORKGROUPS; NOSA_ERR_INVALID otherwise,
 * before any HIP call. */
#define NOSA_MAX_READ_WORKGROUPS 65536
int nosa_hbm_read(const void *src, size_t bytes, int32_t n_workgroups, void *sink,
                  hipStream_t stream);

/* ------------------------------------------------------------ tuning
 * Process-wide launch-shape overrides, for tests and tuning sweeps (host
 * state only; results do not depend on them). value 0 restores the
 * library's choice; the call returns the previous value, or
 * NOSA_ERR_INVALID for an unknown knob or a value outside its range.
 *  NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT  selection entries per decode
 *      workgroup, 4..64. It sets the decode split count and so the decode
 *      workspace size: a call whose workspace was sized before a change
 *      may return NOSA_ERR_WORKSPACE.
 *  NOSA_TUNE_SELECT_SUBS  128-chunk splits scored by one selection
 *      workgroup, 1..2048 (capped at the split count).
 *  NOSA_TUNE_GATHER_VPT  4 KiB pieces of a block that a nosa_fetch_delta_wg
 *      workgroup moves at a time: 1, 2, 4 or 8.
 *  NOSA_TUNE_SELECT_POOL  how a selection's last workgroup finishes: 0 the
 *      library's choice (2 where it applies), 1 the general path (kinds of
 *      every block in LDS, candidates as R per thread, each stage an exact
 *      histogram range refinement, list and eligibility by passes over the
 *      blocks), 2 for a pair of at most 512 candidates, one or two per
 *      thread (up to 256, each stage ranks them: a bitonic sort per wave and
 *      a binary search in each wave's run; above, the range refinement;
 *      kinds, list places and eligibility bits from per-thread flags and
 *      per-wave counts). Both give the same selections.
 * The per-pair arrival counters of the select and decode workspaces sit at
 * the start of each workspace whatever the launch shape, so a change
 * between calls never leaves them on non-zero bytes. */
enum { NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT = 0, NOSA_TUNE_SELECT_SUBS = 1,
       NOSA_TUNE_GATHER_VPT = 2, NOSA_TUNE_SELECT_POOL = 3, NOSA_NUM_TUNE };
int nosa_set_tuning(int knob, int32_t value);

const char *nosa_strerror(int code);
const char *nosa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NOSA_H */
