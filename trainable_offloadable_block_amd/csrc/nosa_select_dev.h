// Device parts of the two-stage block selection (aiwiki "NOSA", How NOSA
// works; NOSA-1B 核心组件揭秘, 核心组件三; l189 article, 2.1), shared by the
// select kernel and the fused append + select kernel: split scoring, and the
// pooling and both top-k stages that the pair's last workgroup runs.
#pragma once

#include "nosa_internal.h"
#include "nosa_lanes.h"
#include "nosa_phase.h"

namespace nosa {
namespace {

// grid_unit for a grid (units per pair, pairs) whose units differ in cost
// by their x index (a pair's scoring splits, its lighter last split and its
// append): each XCD still holds whole pairs, but its dispatch order runs
// over x first (unit x of all its pairs, then unit x + 1): the heavy units
// lead the order and spread over the XCD's CUs before the light ones, where
// the pair-major order stacked up to three scoring splits on some CUs and
// one on others. Pair counts that are not a multiple of 8 keep grid_unit's
// order.
__device__ inline void grid_unit_x_major(int &x, int &y) {
  const int nx = gridDim.x, ny = gridDim.y;
  if ((ny & 7) != 0) {
    grid_unit(x, y);
    return;
  }
  const int L = blockIdx.x + nx * blockIdx.y;
  const int ppx = ny >> 3;                 // pairs per XCD
  const int j = L >> 3;                    // place in XCD (L & 7)'s dispatch order
  x = j / ppx;
  y = (L & 7) * ppx + j % ppx;
}

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

// Heads per chunk in the chunk-weight layout: the group padded to 4, 8 or 16
// so that one 16-byte load never straddles two chunks.
__host__ __device__ inline int padded_group(int G) { return G <= 4 ? 4 : (G <= 8 ? 8 : 16); }

// Device-coherent (agent-scope) stores and loads: how the score workgroups
// of a pair hand their results to the pair's last workgroup without a
// device-scope fence (which would write back the XCD's whole L2).
__device__ inline void put(float *a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float get(const float *a) {
  return __hip_atomic_load(const_cast<float *>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kCoherent = 16;   // buffer-load cache policy: sc1, as the agent-scope loads
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
// LDS (dynamic region) per scoring wave for the transposed chunk weights:
// 32 chunks x 16 heads
constexpr int kScoreTrFloats = 32 * 16;
constexpr size_t kScoreTrBytes = 4 * kScoreTrFloats * sizeof(float);   // 4 waves
// A split's compressed keys staged in the dynamic LDS region on their way
// from coalesced loads to the MFMA operand layout: 128 rows x 256 B (the
// transposes above reuse the region once the products are taken)
constexpr size_t kScoreKeyBytes = (size_t)kChunksPerSplit * kHeadDim * 2;
constexpr size_t kScoreLdsBytes = kScoreKeyBytes > kScoreTrBytes ? kScoreKeyBytes : kScoreTrBytes;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline float4 load4_coherent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent));
}
__device__ inline float2 load2_coherent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kCoherent));
}

// Operands of one split's scoring: the group's query rows as this lane's
// MFMA operands, and the split's stored compressed keys as loaded: thread t
// holds 16-byte words t + 256 j (j < 8) of the split's 128 rows of 256 B.
struct ScoreIn {
  uint4 qv[4], kr[8];
};

// Issues the loads of split `split`'s compressed keys of pair p: each
// instruction reads 4 whole rows (4 KiB over the workgroup), where loads in
// the MFMA layout would read 64 B of each of 16 rows (a streaming read in
// that pattern measured 5.6 against 7.3 TB/s for whole rows). Read once per
// step: non-temporal.
__device__ __forceinline__ void score_load_keys(const Dims &d, const uint16_t *__restrict__ ckey,
                                                int split, int p, ScoreIn &in) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = t + kScoreThreads * j, row = g >> 4, col = g & 15;
    const int chunk = split * kChunksPerSplit + row;
    in.kr[j] = make_uint4(0, 0, 0, 0);
    if (chunk < d.C_max)
      in.kr[j] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(
                                               ckey + ((size_t)p * d.C_max + chunk) * kHeadDim + 8 * col)));
  }
}

// 16-byte slot of (row, column col) of the staged keys: the column is
// XOR-swizzled by a function of the row that is distinct over the 16 rows an
// MFMA operand read touches at once (rows 8 (i / 4) + 4 t + i % 4 of a
// wave's 32), so neither the row-wise writes nor those reads conflict on
// LDS banks.
__device__ inline int key_slot(int row, int col) {
  return row * 16 + (col ^ (((row >> 1) & 12) | (row & 3)));
}

// The loaded keys into the staging area (ks: the dynamic LDS region); row
// skip_row (-1: none) is left to the caller.
__device__ __forceinline__ void keys_to_lds(const ScoreIn &in, uint4 *ks, int skip_row) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = t + kScoreThreads * j, row = g >> 4;
    if (row != skip_row) ks[key_slot(row, g & 15)] = in.kr[j];
  }
}

// This lane's MFMA operands of its wave's 32 rows, from the staging area
// (after a barrier): tile t, k-step s.
__device__ __forceinline__ void keys_from_lds(const uint4 *ks, uint4 (&kv)[2][4]) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) kv[t][s] = ks[key_slot(32 * w + tile_row(h, t), 4 * s + lg)];
}

// Issues the loads of split `split` of pair p. They do not depend on the
// sequence length (rows past it are masked later), so they go out before it
// is known and the kernel waits for one memory round trip.
__device__ __forceinline__ void score_load(const Dims &d, const uint16_t *__restrict__ ckey,
                                           const uint16_t *__restrict__ q, int split, int p,
                                           ScoreIn &in) {
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) in.qv[s] = make_uint4(0, 0, 0, 0);
  if (h < d.G) {
    const uint16_t *qh = q + ((size_t)b * d.Hq + g * d.G + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) in.qv[s] = *reinterpret_cast<const uint4 *>(qh + 32 * s);
  }
  score_load_keys(d, ckey, split, p, in);
}

// Chunks scored by the split workgroups at length L: every complete chunk
// (at most c_pad).
__device__ inline int split_chunks(const Dims &d, int L, int c_pad) {
  return max(min(min(chunks_for(L), d.C_max), c_pad), 0);
}

// The newest chunk's key when the token appended in the same launch completes
// it (the append may still be writing it to memory): built from the key
// ring (the chunk's 31 earlier keys) and the new key, the bits the append
// stores. ring: the pair's [32][128] ring; k_new: the pair's new key; pos:
// the new token's position. Threads t < 128 return dim t.
__device__ inline uint16_t fresh_key_dim(const uint16_t *__restrict__ ring,
                                         const uint16_t *__restrict__ k_new, int pos, int t) {
  const uint16_t kb = k_new[t];
  return mean32_bf16([&](int j) -> uint16_t {
    const int tok = pos - (kPoolKernel - 1) + j;
    return tok == pos ? kb : ring[(tok % kPoolKernel) * kHeadDim + t];
  });
}

// Split `split` of pair p: logits of the group against the split's
// compressed keys among chunks [0, C), published with device-coherent stores.
// fresh_ring: when not NULL, chunk C - 1 was just completed by an append in
// the same launch (position pos, new key fresh_k): the split holding it takes
// that chunk's key from fresh_key_dim instead of memory.
__device__ __forceinline__ void score_compute(const Dims &d, int C, ScoreIn &in, float *ws_e,
                                              float *ws_stats, int c_pad, int n_splits,
                                              int split, int p,
                                              const uint16_t *__restrict__ fresh_ring,
                                              const uint16_t *__restrict__ fresh_k, int pos) {
  const int c0 = split * kChunksPerSplit;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
  const int cg = c0 + 32 * w;
  __shared__ float red_m[4][16], red_z[4][16];
  float *stats = ws_stats + (size_t)2 * (p * n_splits + split) * d.G;   // (M, Z) per head
  if (c0 >= C) {
    if (threadIdx.x < d.G) {
      put(&stats[2 * threadIdx.x], -INFINITY);
      put(&stats[2 * threadIdx.x + 1], 0.0f);
    }
    return;
  }
  extern __shared__ __align__(16) uint8_t score_tr[];
  uint4 *ks = reinterpret_cast<uint4 *>(score_tr);
  const bool fresh_here = fresh_ring && C - 1 < c0 + kChunksPerSplit;   // uniform
  keys_to_lds(in, ks, fresh_here ? C - 1 - c0 : -1);
  if (fresh_here && threadIdx.x < kHeadDim) {
    const int r = C - 1 - c0, dim = threadIdx.x;
    reinterpret_cast<uint16_t *>(&ks[key_slot(r, dim >> 3)])[dim & 7] =
        fresh_key_dim(fresh_ring, fresh_k, pos, dim);
  }
  __syncthreads();
  uint4 kv[2][4];
  keys_from_lds(ks, kv);
  const uint4 (&qv)[4] = in.qv;
  // logits on MFMA; a row past the length only feeds its own (masked) output
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t] = mfma16x16x32(as_bf16x8(kv[t][s]), as_bf16x8(qv[s]), acc[t]);
  }
  // lane (h, lg) now holds head h against chunks cg + 8*lg + m, m = 0..7;
  // logits in the log2 domain, so each weight is one hardware exp2
  const float scale = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)
  float x[8];
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int c = cg + 8 * lg + m;
    x[m] = c < C ? acc[m >> 2][m & 3] * scale : -INFINITY;
    mx = fmaxf(mx, x[m]);
  }
  mx = xor32_max(xor16_max(mx));
  if (lg == 0) red_m[w][h] = mx;
  __syncthreads();
  // the split's first chunk is below C, so M is finite and exp2 of a
  // masked logit (-inf) is 0
  const float M = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
  float ev[8];
  float z = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    ev[m] = __builtin_amdgcn_exp2f(x[m] - M);
    z += ev[m];
  }
  z = xor32_sum(xor16_sum(z));
  if (lg == 0) red_z[w][h] = z;
  const int Gp = padded_group(d.G);
  {
    // the wave's 32 chunks x Gp heads (chunk-major [c][Gp], pad = 0) are one
    // contiguous run of ws_e: transposed through this wave's part of the
    // dynamic LDS, then written as 16-byte device-coherent stores
    float *tr = reinterpret_cast<float *>(score_tr) + w * kScoreTrFloats;   // keys no longer read
    if (h < Gp) {
#pragma unroll
      for (int m = 0; m < 8; ++m) tr[(8 * lg + m) * Gp + h] = h < d.G ? ev[m] : 0.0f;
    }
    asm volatile("" ::: "memory");                // the wave's writes, then its reads (in order)
    const __amdgpu_buffer_rsrc_t er =
        make_rsrc(ws_e + (size_t)p * c_pad * Gp, (uint32_t)(c_pad * Gp * 4));
    const int n4 = 8 * Gp;                        // float4s of the wave's run
    for (int i = l; i < n4; i += 64) {            // uniform trip count per wave
      if (cg + (4 * i) / Gp < C)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4v, *reinterpret_cast<const float4 *>(tr + 4 * i)), er,
            (cg * Gp + 4 * i) * 4, 0, kCoherent);
    }
  }
  __syncthreads();
  if (threadIdx.x < d.G) {
    const int hh = threadIdx.x;
    const float Mh = fmaxf(fmaxf(red_m[0][hh], red_m[1][hh]), fmaxf(red_m[2][hh], red_m[3][hh]));
    const float Zh = (red_z[0][hh] + red_z[1][hh]) + (red_z[2][hh] + red_z[3][hh]);
    put(&stats[2 * hh], Mh);                       // log2 domain, as the weights
    put(&stats[2 * hh + 1], Zh);
  }
}

// Splits ws * subs .. ws * subs + subs - 1 of pair p (those below n_splits),
// one after another: the newest chunk left out (split_chunks). The first
// split's loads go out before the length is used. MULTI = false compiles
// the one-split case alone (subs = 1), without the loop's code.
// k_new: when not NULL, the step's new keys (dev [P][128]) of an append in
// the same launch; a chunk that token completes is then built from the key
// ring (score_compute).
template <bool MULTI>
__device__ __forceinline__ void score_splits(const Dims &d, const nosa_state &st,
                                             const uint16_t *__restrict__ q, int L, float *ws_e,
                                             float *ws_stats, int c_pad, int n_splits, int subs,
                                             int ws, int p,
                                             const uint16_t *__restrict__ k_new = nullptr) {
  const int split0 = MULTI ? ws * subs : ws;       // < n_splits: ceil(n_splits / subs) groups
  ScoreIn in;
  score_load(d, st.ckey, q, split0, p, in);
  const int C = split_chunks(d, L, c_pad);
  const bool fresh = k_new != nullptr && L >= kPoolKernel && (L - kPoolKernel) % kPoolStride == 0 &&
                     C == chunks_for(L);
  const uint16_t *fring = fresh ? st.tail_keys + (size_t)p * kPoolKernel * kHeadDim : nullptr;
  const uint16_t *fk = fresh ? k_new + (size_t)p * kHeadDim : nullptr;
  score_compute(d, C, in, ws_e, ws_stats, c_pad, n_splits, split0, p, fring, fk, L - 1);
  if (!MULTI) return;
  for (int j = 1; j < subs; ++j) {                 // uniform
    const int split = split0 + j;
    if (split >= n_splits) break;
    __syncthreads();                               // the last split's reductions are read
    score_load_keys(d, st.ckey, split, p, in);     // the query rows stay
    score_compute(d, C, in, ws_e, ws_stats, c_pad, n_splits, split, p, fring, fk, L - 1);
  }
}

// ---- workgroup top-k on 64-bit composite keys ----------------------------
// A key is (order_key(score) << 32) | ~block: larger score first, then the
// lower block id; keys are distinct and 0 marks "not a candidate".

__device__ inline uint64_t compose_key(float score, int blk) {
  return (static_cast<uint64_t>(order_key(score)) << 32) |
         static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(blk));
}

// DPP lane exchange inside a row of 16 lanes: xor 1, xor 2 (quad
// permutations), then the mirrors of 8 and 16 lanes; for min / max / sum
// any pairing that joins the two halves serves.
template <int CTRL>
__device__ inline uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t v) {
  return (static_cast<uint64_t>(dpp32<CTRL>(static_cast<uint32_t>(v >> 32))) << 32) |
         dpp32<CTRL>(static_cast<uint32_t>(v));
}
template <int CTRL>
__device__ inline void row_step(uint64_t &mn, uint64_t &mx, uint32_t &c) {
  const uint64_t a = dpp64<CTRL>(mn), b = dpp64<CTRL>(mx);
  mn = a < mn ? a : mn;
  mx = b > mx ? b : mx;
  c += dpp32<CTRL>(c);
}

__device__ inline uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes: DPP row shifts inside each row of
// 16 lanes, then the row totals (lanes 15, 31, 47) carried forward.
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  x += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x111, 0xF, 0xF, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x112, 0xF, 0xF, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x114, 0xF, 0xF, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x118, 0xF, 0xF, true));
  const uint32_t r0 = __builtin_amdgcn_readlane(static_cast<int>(x), 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(static_cast<int>(x), 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(static_cast<int>(x), 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

constexpr int kTopkBits = 8, kTopkBins = 1 << kTopkBits;   // bins per refinement round

constexpr int kSmallWords = 32;   // eligibility words <= 512 consecutive candidates touch (<= 17)

struct __align__(16) TopkLds {
  uint32_t hist[2][kTopkBins];
  uint64_t mn[2][kTopkThreads / 64], mx[2][kTopkThreads / 64];
  uint32_t cnt[2][kTopkThreads / 64];
  uint32_t clr[kSmallWords];   // eligibility bits finish_select_small clears, zero at entry
};

// Zeroes a TopkLds's histograms and clear marks (thread t of kTopkThreads);
// the caller's next barrier orders it before their use.
__device__ inline void topk_lds_init(TopkLds &tk) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kTopkBins / kTopkThreads; ++i) {
    tk.hist[0][t + kTopkThreads * i] = 0;
    tk.hist[1][t + kTopkThreads * i] = 0;
  }
  if (t < kSmallWords) tk.clr[t] = 0;
}

// Calls mark(r) in thread t for each of the k largest nonzero keys of the
// NT-thread workgroup (thread t holds the keys of candidates t + NT r, r < R;
// a thread marks only its own keys) and returns the rounds it ran.
// Exact selection by range refinement: each round histograms the active keys
// into 256 bins over [min, max] (the top 8 bits of their spread), keeps every
// key above the bin holding the k-th largest, drops those below it, and goes
// on inside that bin; a bin whose keys are all wanted ends it. The spread
// shrinks by 8 bits per round, so 64-bit keys need at most 8 rounds.
// hist[0] must be zero on entry; both are zero again on return. Called by
// all threads; the caller syncs before another thread reads a mark.
template <int R, int NT = kTopkThreads, typename Mark>
__device__ __forceinline__ int wg_topk_marks(const uint64_t (&key)[R], int k, Mark mark, TopkLds &sh,
                                             int clk_p = 0, int clk_slot = -1) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  bool act[R];
#pragma unroll
  for (int r = 0; r < R; ++r) act[r] = key[r] != 0;
  int need = k;
  int rounds = 0;
  for (int round = 0; need > 0 && round < 9; ++round) {    // uniform; <= 8 refinements
    ++rounds;
    const int par = round & 1;
    uint64_t mn = ~0ull, mx = 0;
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (act[r]) {
        mn = key[r] < mn ? key[r] : mn;
        mx = key[r] > mx ? key[r] : mx;
        ++c;
      }
    row_step<0xB1>(mn, mx, c);            // quad_perm [1,0,3,2]
    row_step<0x4E>(mn, mx, c);            // quad_perm [2,3,0,1]
    row_step<0x141>(mn, mx, c);           // row_half_mirror
    row_step<0x140>(mn, mx, c);           // row_mirror
    {
      uint64_t wm = readlane_u64(mn, 0), wx = readlane_u64(mx, 0);
      uint32_t wc = __builtin_amdgcn_readlane(static_cast<int>(c), 0);
#pragma unroll
      for (int row = 1; row < 4; ++row) {
        const uint64_t a = readlane_u64(mn, 16 * row), b = readlane_u64(mx, 16 * row);
        wm = a < wm ? a : wm;
        wx = b > wx ? b : wx;
        wc += __builtin_amdgcn_readlane(static_cast<int>(c), 16 * row);
      }
      if (lane == 0) {
        sh.mn[par][w] = wm;
        sh.mx[par][w] = wx;
        sh.cnt[par][w] = wc;
      }
    }
    __syncthreads();
    if (clk_slot == 12 && round == 0) NOSA_PHASE(clk_p, kPhasePoolRow, 1);
#pragma unroll
    for (int i = 0; i < kTopkBins / NT; ++i)         // next round's bins
      sh.hist[par ^ 1][t + NT * i] = 0;
    mn = ~0ull;
    mx = 0;
    c = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const uint64_t a = sh.mn[par][i], b = sh.mx[par][i];
      mn = a < mn ? a : mn;
      mx = b > mx ? b : mx;
      c += sh.cnt[par][i];
    }
    if (c <= static_cast<uint32_t>(need)) {                  // uniform: take them all
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (act[r]) mark(r);
      break;
    }
    const int span = mx > mn ? 64 - __builtin_clzll(mx - mn) : 0;   // c >= 2 distinct keys
    const int shift = span > kTopkBits ? span - kTopkBits : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (act[r]) atomicAdd(&sh.hist[par][(key[r] - mn) >> shift], 1u);
    __syncthreads();
    if (clk_slot == 12 && round == 0) NOSA_PHASE(clk_p, kPhasePoolRow, 2);
    // bin holding the need-th largest: lane l sums the BPL bins below
    // kTopkBins - BPL l, a prefix over lanes counts from the top
    constexpr int BPL = kTopkBins / 64;
    uint32_t hb[BPL], s4 = 0;
    {
      const uint4 *hv = reinterpret_cast<const uint4 *>(&sh.hist[par][kTopkBins - BPL * (lane + 1)]);
#pragma unroll
      for (int i = 0; i < BPL / 4; ++i) {
        const uint4 v = hv[BPL / 4 - 1 - i];     // descending bin order
        hb[4 * i] = v.w;
        hb[4 * i + 1] = v.z;
        hb[4 * i + 2] = v.y;
        hb[4 * i + 3] = v.x;
      }
#pragma unroll
      for (int i = 0; i < BPL; ++i) s4 += hb[i];
    }
    const uint32_t incl = wave_incl_scan(s4);
    const uint64_t hit = __ballot(incl >= static_cast<uint32_t>(need));
    const int ls = __builtin_ctzll(hit);                     // exists: total c > need
    int bstar = 0;
    uint32_t above = incl - s4, inbin = 0;
    {
      bool found = false;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        if (!found && above + hb[i] >= static_cast<uint32_t>(need)) {
          bstar = kTopkBins - 1 - BPL * lane - i;
          inbin = hb[i];
          found = true;
        } else if (!found) {
          above += hb[i];
        }
      }
    }
    bstar = __builtin_amdgcn_readlane(bstar, ls);
    above = __builtin_amdgcn_readlane(static_cast<int>(above), ls);
    inbin = __builtin_amdgcn_readlane(static_cast<int>(inbin), ls);
    const int rest = need - static_cast<int>(above);
    const bool all_in = inbin == static_cast<uint32_t>(rest);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (act[r]) {
        const int bin = static_cast<int>((key[r] - mn) >> shift);
        if (bin > bstar || (bin == bstar && all_in)) {
          mark(r);
          act[r] = false;
        } else if (bin < bstar) {
          act[r] = false;
        }
      }
    if (clk_slot == 12 && round == 0) NOSA_PHASE(clk_p, kPhasePoolRow, 3);
    if (all_in) break;                                       // uniform
    need = rest;
  }
  if (clk_slot >= 0) NOSA_PHASE_VAL(clk_p, kPhasePoolRow, clk_slot, rounds);
  // leave both histograms zero for the next call
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTopkBins / NT; ++i) {
    sh.hist[0][t + NT * i] = 0;
    sh.hist[1][t + NT * i] = 0;
  }
  return rounds;
}

// wg_topk_marks that marks kind[bb0 + t + NT r] = val.
template <int R, int NT = kTopkThreads>
__device__ __forceinline__ void wg_topk(const uint64_t (&key)[R], int k, int bb0, uint8_t *kind,
                                        uint8_t val, TopkLds &sh, int clk_p = 0,
                                        int clk_slot = -1) {
  wg_topk_marks<R, NT>(key, k, [&](int r) { kind[bb0 + threadIdx.x + NT * r] = val; }, sh, clk_p,
                       clk_slot);
}

// Query-aware score of block bb: max over its overlapping chunks
// 4bb-1 .. 4bb+3 of the chunk score a_c.
// (C >= 1; the five reads are unconditional, at clamped indices, so they
// go out together)
__device__ inline float block_qscore(const float *a_sh, int bb, int C) {
  float v[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) v[j] = a_sh[min(max(4 * bb - 1 + j, 0), C - 1)];
  float qb = -INFINITY;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int c = 4 * bb - 1 + j;
    qb = (c >= 0 && c < C) ? fmaxf(qb, v[j]) : qb;
  }
  return qb;
}

// Both selection stages with R candidate slots per thread (candidate
// t + 256 r, block n_sink + t + 256 r). Stage 1: the k_q candidates of
// highest query-aware score; stage 2: the k_e' eligible candidates of highest
// agnostic score among the rest. Once decoding is under way the eligible
// candidates left after stage 1 rarely outnumber k_e' (the eligible set only
// keeps blocks selected at the previous step), and then stage 2 takes them
// all without ranking.
template <int R>
__device__ __forceinline__ void select_stages(const Dims &d, int p, int n_cand, int C, bool do_q, bool do_e,
                              const float *a_sh, const uint32_t *el_sh, const float *be,
                              float e0, uint8_t *kind, float *dbg, TopkLds &tk) {
  __shared__ int n_rank_sh[kTopkThreads / 64];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (do_q) {
    uint64_t kq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + kTopkThreads * r, bb = d.n_sink + i;
      kq[r] = 0;
      if (i < n_cand) {
        const float qb = block_qscore(a_sh, bb, C);
        kq[r] = compose_key(qb, bb);
        if (dbg) dbg[(size_t)p * d.NB_max + bb] = qb;
      }
    }
    // returns after a barrier that follows its marks of kind[]
    NOSA_PHASE(p, kPhasePoolRow, 0);
    wg_topk(kq, d.k_q, d.n_sink, kind, NOSA_KIND_QUERY, tk, p, 12);
  }
  NOSA_PHASE(p, kPhasePoolRow, 7);
  if (do_e) {
    uint64_t ke[R];
    int c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + kTopkThreads * r, bb = d.n_sink + i;
      ke[r] = 0;
      if (i < n_cand && ((el_sh[bb >> 5] >> (bb & 31)) & 1u) && kind[bb] != NOSA_KIND_QUERY)
        ke[r] = compose_key(r == 0 ? e0 : get(&be[bb]), bb);
      c += __popcll(__ballot(ke[r] != 0));
    }
    if (lane == 0) n_rank_sh[w] = c;
    __syncthreads();
    int n_rank = 0;
#pragma unroll
    for (int ww = 0; ww < kTopkThreads / 64; ++ww) n_rank += n_rank_sh[ww];
    NOSA_PHASE_VAL(p, kPhasePoolRow, 14, n_rank);
    if (n_rank <= d.k_e_dyn) {                                  // uniform: take them all
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (ke[r] != 0) kind[d.n_sink + t + kTopkThreads * r] = NOSA_KIND_AGNOSTIC;
      NOSA_PHASE_VAL(p, kPhasePoolRow, 13, 0);
    } else {
      wg_topk(ke, d.k_e_dyn, d.n_sink, kind, NOSA_KIND_AGNOSTIC, tk, p, 13);
    }
  }
}

// 32-bit value of lane (lane ^ D) of the wave for D = 1, 2, 4, 8, on DPP:
// quad permutations for 1 and 2; a row rotation by 8 (within a row of 16
// lanes it is the xor); for 4, a shift by 4 either way within the row, each
// lane taking the one that stays inside its group of 8.
template <int D>
__device__ inline uint32_t xor_lane_dpp(uint32_t v, int lane) {
  const int x = static_cast<int>(v);
  if constexpr (D == 4) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);    // row_shl:4, lane + 4
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);    // row_shr:4, lane - 4
    return static_cast<uint32_t>((lane & 4) ? dn : up);
  } else {
    constexpr int ctrl = D == 1 ? 0xB1 : (D == 2 ? 0x4E : 0x128);        // quad_perm / row_ror:8
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, ctrl, 0xF, 0xF, true));
  }
}

// One compare-exchange step of a bitonic network over the wave's lanes: the
// lane keeps the larger of its key and lane (lane ^ D)'s when it is the
// lower lane of a descending block of K lanes or the upper lane of an
// ascending one. D = 16 and 32 use the permlane swaps, which hand each lane
// both keys of its pair (the same pair order for both words of a key), so
// the lane keeps their larger or smaller one.
template <int K, int D>
__device__ inline uint64_t bitonic_step(uint64_t v, int lane) {
  const bool keep_larger = ((lane & D) == 0) == ((lane & K) == 0);
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  if constexpr (D <= 8) {
    const uint64_t o = (static_cast<uint64_t>(xor_lane_dpp<D>(hi, lane)) << 32) |
                       xor_lane_dpp<D>(lo, lane);
    return (v > o) == keep_larger ? v : o;
  } else {
    const auto h = D == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                           : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l = D == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                           : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const uint64_t a = (static_cast<uint64_t>(h[0]) << 32) | l[0];
    const uint64_t b = (static_cast<uint64_t>(h[1]) << 32) | l[1];
    return (a > b) == keep_larger ? a : b;
  }
}

// The wave's 64 keys (one per lane) in descending order: a bitonic network
// of 21 compare-exchange steps on cross-lane moves.
__device__ __forceinline__ uint64_t wave_sort64(uint64_t v, int lane) {
  v = bitonic_step<2, 1>(v, lane);
  v = bitonic_step<4, 2>(v, lane);
  v = bitonic_step<4, 1>(v, lane);
  v = bitonic_step<8, 4>(v, lane);
  v = bitonic_step<8, 2>(v, lane);
  v = bitonic_step<8, 1>(v, lane);
  v = bitonic_step<16, 8>(v, lane);
  v = bitonic_step<16, 4>(v, lane);
  v = bitonic_step<16, 2>(v, lane);
  v = bitonic_step<16, 1>(v, lane);
  v = bitonic_step<32, 16>(v, lane);
  v = bitonic_step<32, 8>(v, lane);
  v = bitonic_step<32, 4>(v, lane);
  v = bitonic_step<32, 2>(v, lane);
  v = bitonic_step<32, 1>(v, lane);
  v = bitonic_step<64, 32>(v, lane);
  v = bitonic_step<64, 16>(v, lane);
  v = bitonic_step<64, 8>(v, lane);
  v = bitonic_step<64, 4>(v, lane);
  v = bitonic_step<64, 2>(v, lane);
  return bitonic_step<64, 1>(v, lane);
}

// Rank of thread t's key among the workgroup's kTopkThreads keys, one per
// thread (distinct where nonzero; zero keys are below every other key): the
// number of keys above it. Each wave sorts its 64 keys in descending order
// (wave_sort64) and writes them to srt (LDS, kTopkThreads entries) as one
// run; after one barrier each thread counts the keys above its own in every
// run by binary lifting (7 dependent reads, the four runs at once). A fixed
// cost whatever the keys, where a range refinement's rounds depend on how
// they spread and tie (with two keys per thread, merging each wave's two
// sorted runs and searching runs of 128 measured slower than the
// refinement: 2.4 against 1.9 us at 32K). The caller syncs before srt is
// written again. Called by all threads, with every lane of each wave active
// (the network moves values between lanes).
__device__ __forceinline__ uint32_t wg_rank256(uint64_t key, uint64_t *srt) {
  constexpr int NR = kTopkThreads / 64;            // runs, one per wave
  const int t = threadIdx.x, lane = t & 63;
  srt[t] = wave_sort64(key, lane);                 // run w: srt[64 w .. 64 w + 63]
  __syncthreads();
  // per run, the number of keys above `key` by binary lifting: pos grows by
  // each power of two whose last key is still above (indices stay <= 62),
  // then by one if the key at pos is (a run whose 64 keys are all above)
  uint32_t pos[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) pos[q] = 0;
#pragma unroll
  for (int step = 32; step >= 1; step >>= 1) {
    uint64_t m[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) m[q] = srt[64 * q + pos[q] + step - 1];
#pragma unroll
    for (int q = 0; q < NR; ++q) pos[q] += m[q] > key ? step : 0;
  }
  uint32_t above = 0;
#pragma unroll
  for (int q = 0; q < NR; ++q) above += pos[q] + (srt[64 * q + pos[q]] > key ? 1u : 0u);
  return above;
}

// ORs a wave's 64-lane mask of blocks base .. base + 63 into the eligibility
// clear words clr[word - w_lo] (at most three words; lane 0 does it, one LDS
// atomic per word touched).
__device__ inline void mark_clear(uint64_t m, int base, int w_lo, uint32_t *clr) {
  if ((threadIdx.x & 63) != 0 || m == 0) return;
  const int wd0 = base >> 5, sh = base & 31;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    // bits of word wd0 + i: blocks 32 (wd0 + i) .. + 31, i.e. mask bits
    // 32 i - sh .. 32 i - sh + 31
    const int lo = 32 * i - sh;
    const uint64_t part = lo >= 0 ? (lo < 64 ? m >> lo : 0ull) : m << (-lo);
    const uint32_t bits = static_cast<uint32_t>(part);
    if (bits) atomicOr(&clr[wd0 + i - w_lo], bits);
  }
}

// Both stages, the ascending selection list and the eligibility update of
// pair p when it has at most R * kTopkThreads candidates (R = 1 or 2):
// thread t owns candidates t + 256 r, blocks n_sink + t + 256 r (none past
// n_cand), so a block's kind, its place in the list and its eligibility bit
// need no LDS array of kinds and no pass over the blocks. kq: their stage-1
// keys (0 unless stage 1 runs); e0: candidate t's agnostic score (the others'
// are read from be if stage 2 ranks); el_sh: the eligibility words as they
// stand; tk.clr zero (topk_lds_init, then a barrier). With one candidate per
// thread each stage keeps the candidates with fewer than k keys above their
// own (wg_rank256: the keys are distinct, so these are exactly the sets a
// range refinement keeps); with two, each stage is that range refinement
// (wg_topk_marks). Stage 2 takes every eligible candidate stage 1 left when
// they do not outnumber k_e', as select_stages does. The list holds the sink blocks, the kept
// candidates, then the window blocks (ascending block order), cut at k.
// Called by all threads.
template <int R>
__device__ __forceinline__ void finish_select_small(const Dims &d, const nosa_state &st, int p,
                                                    int nb, int win_lo, int n_cand, bool do_q,
                                                    bool do_e, const uint64_t (&kq)[R],
                                                    float e0, const float *be,
                                                    const uint32_t *el_sh, int32_t *sel,
                                                    int32_t *n_sel, uint8_t *kind_out,
                                                    TopkLds &tk) {
  constexpr int NW = kTopkThreads / 64;
  __shared__ int cnt_sh[2][R][NW];
  __shared__ uint64_t srt[R == 1 ? kTopkThreads : 1];   // wg_rank256's runs
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int w_lo = d.n_sink >> 5;
  int bb[R];
  bool cand[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    bb[r] = d.n_sink + t + kTopkThreads * r;
    cand[r] = t + kTopkThreads * r < n_cand;
  }
  // 1. stage 1: the k_q candidates of highest query-aware score
  bool in_q[R];
#pragma unroll
  for (int r = 0; r < R; ++r) in_q[r] = false;
  if (do_q) {                                      // uniform
    if constexpr (R == 1) {
      const uint32_t rank = wg_rank256(kq[0], srt);   // every thread takes part
      in_q[0] = kq[0] != 0 && rank < static_cast<uint32_t>(d.k_q);
    } else {
      wg_topk_marks<R>(kq, d.k_q, [&](int r) { in_q[r] = true; }, tk, p, 12);
    }
  }
  NOSA_PHASE(p, kPhasePoolRow, 7);
  // 2. stage 2 over the eligible candidates stage 1 left; the candidates the
  // list keeps and those it leaves out are counted and marked as if stage 2
  // took them all (the usual case), completed below otherwise
  bool e_cand[R], inc[R];
  uint64_t m_in[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    e_cand[r] = do_e && cand[r] && !in_q[r] && ((el_sh[bb[r] >> 5] >> (bb[r] & 31)) & 1u);
    inc[r] = in_q[r] || e_cand[r];
    mark_clear(__ballot(cand[r] && !inc[r]), d.n_sink + kTopkThreads * r + 64 * w, w_lo, tk.clr);
    const uint64_t m_e = __ballot(e_cand[r]);
    m_in[r] = __ballot(inc[r]);
    if (lane == 0) {
      cnt_sh[0][r][w] = __popcll(m_e);
      cnt_sh[1][r][w] = __popcll(m_in[r]);
    }
  }
  __syncthreads();
  int n_rank = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) n_rank += cnt_sh[0][r][ww];
  NOSA_PHASE_VAL(p, kPhasePoolRow, 14, n_rank);
  int row = 1;
  if (n_rank > d.k_e_dyn) {                        // uniform: rank them by agnostic score
    uint64_t ke[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      ke[r] = e_cand[r] ? compose_key(r == 0 ? e0 : get(&be[bb[r]]), bb[r]) : 0;
    bool sel_e[R];
    if constexpr (R == 1) {
      const uint32_t rank = wg_rank256(ke[0], srt);   // srt's reads ended before the barrier
      sel_e[0] = ke[0] != 0 && rank < static_cast<uint32_t>(d.k_e_dyn);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) sel_e[r] = false;
      wg_topk_marks<R>(ke, d.k_e_dyn, [&](int r) { sel_e[r] = true; }, tk);
    }
    NOSA_PHASE_VAL(p, kPhasePoolRow, 13, 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool in_e = sel_e[r];
      // the marks so far leave out the candidates stage 2 could have taken;
      // add those it drops (no one has read the marks yet)
      mark_clear(__ballot(e_cand[r] && !in_e), d.n_sink + kTopkThreads * r + 64 * w, w_lo,
                 tk.clr);
      inc[r] = in_q[r] || in_e;
      m_in[r] = __ballot(inc[r]);
      if (lane == 0) cnt_sh[0][r][w] = __popcll(m_in[r]);   // n_rank's reads ended before a barrier
    }
    __syncthreads();
    row = 0;
  } else {
    NOSA_PHASE_VAL(p, kPhasePoolRow, 13, 0);
  }
  NOSA_PHASE(p, kPhasePoolRow, 8);
  // 3. ascending selection list: sinks, kept candidates, window
  const int n_s = min(d.n_sink, nb), n_w = max(0, nb - win_lo);
  int32_t *sp = sel + (size_t)p * d.k;
  uint8_t *kp = kind_out ? kind_out + (size_t)p * d.k : nullptr;
  int kept = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int off = __popcll(m_in[r] & ((1ull << lane) - 1ull)), kept_r = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (ww < w) off += cnt_sh[row][r][ww];
      kept_r += cnt_sh[row][r][ww];
    }
    const int pos = n_s + kept + off;
    if (inc[r] && pos < d.k) {
      sp[pos] = bb[r];
      if (kp) kp[pos] = in_q[r] ? NOSA_KIND_QUERY : NOSA_KIND_AGNOSTIC;
    }
    kept += kept_r;
  }
  const int tot = n_s + kept + n_w;
  for (int j = t; j < n_s + n_w; j += kTopkThreads) {   // the sink and window blocks
    const bool sink = j < n_s;
    const int pos = sink ? j : j + kept;
    if (pos < d.k) {
      sp[pos] = sink ? j : win_lo + (j - n_s);
      if (kp) kp[pos] = sink ? NOSA_KIND_SINK : NOSA_KIND_WINDOW;
    }
  }
  for (int j = tot + t; j < d.k; j += kTopkThreads) {
    sp[j] = -1;
    if (kp) kp[j] = NOSA_KIND_NONE;
  }
  if (t == 0) n_sel[p] = min(tot, d.k);
  NOSA_PHASE(p, kPhasePoolRow, 9);
  // 4. eligibility: a candidate outside the selection is out for good
  if (n_cand > 0 && t < kSmallWords) {
    const int wd = w_lo + t;
    const uint32_t clear = tk.clr[t];
    if (clear) st.eligible[(size_t)p * d.elig_words + wd] = el_sh[wd] & ~clear;
  }
  NOSA_PHASE(p, kPhasePoolRow, 10);
}

constexpr int kMaxCandPerThread = (kMaxContext / kBlock) / kTopkThreads;   // 16
constexpr int kLoadBatch = 10;    // chunk-weight float4 loads in flight per thread
constexpr int kStatBatches = 4;   // split statistics loaded early: 16 splits each

// Both stages, the ascending selection list and the eligibility update of
// pair p at a length with nb blocks, once the chunk scores a_sh[0, C), the
// eligibility words el_sh and the kinds of the sink and window blocks sit in
// LDS (kind[] of every other block NOSA_KIND_NONE); e0 is candidate t's
// agnostic score, loaded early. Called by all threads.
__device__ __forceinline__ void finish_select(const Dims &d, const nosa_state &st, int p, int nb,
                                              int win_lo, int n_cand, int C, bool do_q,
                                              bool do_e, const float *a_sh,
                                              const uint32_t *el_sh, const float *be, float e0,
                                              uint8_t *kind, int32_t *sel, int32_t *n_sel,
                                              uint8_t *kind_out, float *dbg, TopkLds &tk) {
  __shared__ int cnt_sh[2][kTopkThreads / 64];
  const int t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  if (d.pool_small && n_cand <= 2 * kTopkThreads) {   // uniform: a candidate or two per thread
    uint64_t kq[2] = {0, 0};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int bb = d.n_sink + t + kTopkThreads * r;
      if (do_q && t + kTopkThreads * r < n_cand) {
        const float qb = block_qscore(a_sh, bb, C);
        kq[r] = compose_key(qb, bb);
        if (dbg) dbg[(size_t)p * d.NB_max + bb] = qb;
      }
    }
    NOSA_PHASE(p, kPhasePoolRow, 0);
    if (n_cand <= kTopkThreads) {
      const uint64_t k1[1] = {kq[0]};
      finish_select_small<1>(d, st, p, nb, win_lo, n_cand, do_q, do_e, k1, e0, be, el_sh, sel,
                             n_sel, kind_out, tk);
    } else {
      finish_select_small<2>(d, st, p, nb, win_lo, n_cand, do_q, do_e, kq, e0, be, el_sh, sel,
                             n_sel, kind_out, tk);
    }
    return;
  }
  // 3. both stages, with as many candidate slots per thread as needed
  {
    const int m = (n_cand + kTopkThreads - 1) / kTopkThreads;   // <= kMaxCandPerThread
    if (m <= 1)
      select_stages<1>(d, p, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, dbg, tk);
    else if (m <= 2)
      select_stages<2>(d, p, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, dbg, tk);
    else if (m <= 4)
      select_stages<4>(d, p, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, dbg, tk);
    else if (m <= 8)
      select_stages<8>(d, p, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, dbg, tk);
    else
      select_stages<kMaxCandPerThread>(d, p, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind,
                                       dbg, tk);
  }
  __syncthreads();
  NOSA_PHASE(p, kPhasePoolRow, 8);

  // 4. ascending selection list: ballot + prefix count per 256 blocks (up
  // to 512 blocks, two adjacent blocks per thread and one prefix)
  if (nb <= 2 * kTopkThreads) {                                       // uniform
    int32_t *sp = sel + (size_t)p * d.k;
    uint8_t *kp = kind_out ? kind_out + (size_t)p * d.k : nullptr;
    const int b0 = 2 * t;
    const uint8_t k0 = b0 < nb ? kind[b0] : (uint8_t)NOSA_KIND_NONE;
    const uint8_t k1 = b0 + 1 < nb ? kind[b0 + 1] : (uint8_t)NOSA_KIND_NONE;
    const int mine = (k0 != NOSA_KIND_NONE ? 1 : 0) + (k1 != NOSA_KIND_NONE ? 1 : 0);
    const uint32_t incl = wave_incl_scan(static_cast<uint32_t>(mine));
    if (lane == 63) cnt_sh[0][w] = static_cast<int>(incl);
    __syncthreads();
    int off = static_cast<int>(incl) - mine, tot = 0;
#pragma unroll
    for (int ww = 0; ww < kTopkThreads / 64; ++ww) {
      if (ww < w) off += cnt_sh[0][ww];
      tot += cnt_sh[0][ww];
    }
    if (k0 != NOSA_KIND_NONE) {
      if (off < d.k) {
        sp[off] = b0;
        if (kp) kp[off] = k0;
      }
      ++off;
    }
    if (k1 != NOSA_KIND_NONE && off < d.k) {
      sp[off] = b0 + 1;
      if (kp) kp[off] = k1;
    }
    for (int j = tot + t; j < d.k; j += kTopkThreads) {
      sp[j] = -1;
      if (kp) kp[j] = NOSA_KIND_NONE;
    }
    if (t == 0) n_sel[p] = min(tot, d.k);
  } else {
    int32_t *sp = sel + (size_t)p * d.k;
    uint8_t *kp = kind_out ? kind_out + (size_t)p * d.k : nullptr;
    int running = 0;
    for (int base = 0; base < nb; base += kTopkThreads) {            // uniform
      const int bb = base + t;
      const bool in = bb < nb && kind[bb] != NOSA_KIND_NONE;
      const uint64_t mask = __ballot(in);
      const int below = __popcll(mask & ((1ull << lane) - 1ull));
      if (lane == 0) cnt_sh[(base / kTopkThreads) & 1][w] = __popcll(mask);
      __syncthreads();
      const int *cs = cnt_sh[(base / kTopkThreads) & 1];
      int off = running, tot = 0;
#pragma unroll
      for (int ww = 0; ww < kTopkThreads / 64; ++ww) {
        if (ww < w) off += cs[ww];
        tot += cs[ww];
      }
      off += below;
      if (in && off < d.k) {
        sp[off] = bb;
        if (kp) kp[off] = kind[bb];
      }
      running += tot;
    }
    for (int j = running + t; j < d.k; j += kTopkThreads) {
      sp[j] = -1;
      if (kp) kp[j] = NOSA_KIND_NONE;
    }
    if (t == 0) n_sel[p] = min(running, d.k);
  }
  NOSA_PHASE(p, kPhasePoolRow, 9);

  // 5. eligibility: a candidate outside the selection is out for good
  if (n_cand > 0) {
    uint32_t *el = st.eligible + (size_t)p * d.elig_words;
    for (int base = 64 * w; base < win_lo; base += kTopkThreads) {   // wave-uniform
      const int bb = base + lane;
      const bool out = bb >= d.n_sink && bb < win_lo && kind[bb] == NOSA_KIND_NONE;
      const uint64_t mask = __ballot(out);
      const uint32_t clear = static_cast<uint32_t>(mask >> (lane & 32));
      if ((lane & 31) == 0 && clear) el[bb >> 5] = el_sh[bb >> 5] & ~clear;
    }
  }
  NOSA_PHASE(p, kPhasePoolRow, 10);
}

// Chunk scores of one batch of chunk-weight float4s (eb[u] = float4 k0 + t +
// 256 u of the chunk-major [c][GP] array): each lane takes the dot product
// of its 4 heads with their split factors, the GP / 4 adjacent lanes of a
// chunk add theirs with DPP quad exchanges, and the chunk's first lane
// stores a_c. Branch-free up to the stores, so the LDS reads of all of a
// thread's float4s go out together.
template <int GP>
__device__ __forceinline__ void chunk_scores(const float4 (&eb)[kLoadBatch], int k0, int n4,
                                             int n_splits, const float *f_sh, float *a_sh) {
  constexpr int LPC = GP / 4;                    // lanes per chunk: 1, 2, 4
  constexpr int kHalf = kLoadBatch / 2;          // float4s whose factors are read together
  const int t = threadIdx.x;
#pragma unroll
  for (int u0 = 0; u0 < kLoadBatch; u0 += kHalf) {
    float a[kHalf];
#pragma unroll
    for (int v = 0; v < kHalf; ++v) {
      const int u = u0 + v;
      const int k4 = k0 + t + kTopkThreads * u;
      const int c = k4 / LPC, h0 = 4 * (k4 % LPC);
      const int split = min(c / kChunksPerSplit, n_splits - 1);
      const float4 f = *reinterpret_cast<const float4 *>(f_sh + split * GP + h0);
      float x = eb[u].x * f.x;
      x = fmaf(eb[u].y, f.y, x);
      x = fmaf(eb[u].z, f.z, x);
      a[v] = fmaf(eb[u].w, f.w, x);
    }
#pragma unroll
    for (int v = 0; v < kHalf; ++v) {
      if (LPC >= 2) a[v] += dpp_f32<0xB1>(a[v]);   // lane ^ 1
      if (LPC >= 4) a[v] += dpp_f32<0x4E>(a[v]);   // lane ^ 2
    }
#pragma unroll
    for (int v = 0; v < kHalf; ++v) {
      const int k4 = k0 + t + kTopkThreads * (u0 + v);
      if (k4 < n4 && k4 % LPC == 0) a_sh[k4 / LPC] = a[v];
    }
  }
}

// Pooling's first step: per-split factors exp(m_split - M) / Z (the maxima
// in the log2 domain, so one hardware exp2 each) of each
// head's softmax over all complete chunks (0 for the padding heads), into
// f_sh[split][Gp]. Thread (t / 16, t % 16) takes head t / 16's statistics
// of splits t % 16 + 16 i; stv_raw holds the first kStatBatches of them,
// loaded early. Ends with a barrier.
__device__ __forceinline__ void pool_factors(const Dims &d, int Gp, int used, bool do_q,
                                             __amdgpu_buffer_rsrc_t sr,
                                             const float2 (&stv_raw)[kStatBatches], float *f_sh) {
  const int t = threadIdx.x;
  const int sh_h = t >> 4, sh_j = t & 15;
  if (do_q && sh_h < Gp) {
    const bool real = sh_h < d.G;
    constexpr int kPre = 16 * kStatBatches;          // splits held in registers
    float2 sv[kStatBatches];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStatBatches; ++i) {
      sv[i] = (real && sh_j + 16 * i < used) ? stv_raw[i] : make_float2(-INFINITY, 0.0f);
      m = fmaxf(m, sv[i].x);
    }
    if (real)
      for (int s = sh_j + kPre; s < used; s += 16) m = fmaxf(m, load2_coherent(sr, 8 * (s * d.G + sh_h)).x);
    m = row16_max(m);
    float es[kStatBatches];
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < kStatBatches; ++i) {
      es[i] = sv[i].y > 0.0f ? __builtin_amdgcn_exp2f(sv[i].x - m) : 0.0f;
      z += sv[i].y * es[i];
    }
    if (real)
      for (int s = sh_j + kPre; s < used; s += 16) {
        const float2 v = load2_coherent(sr, 8 * (s * d.G + sh_h));
        if (v.y > 0.0f) z += v.y * __builtin_amdgcn_exp2f(v.x - m);
      }
    z = row16_sum(z);
    const float rz = real ? 1.0f / z : 0.0f;
#pragma unroll
    for (int i = 0; i < kStatBatches; ++i)
      if (sh_j + 16 * i < used) f_sh[(sh_j + 16 * i) * Gp + sh_h] = es[i] * rz;
    for (int s = sh_j + kPre; s < used; s += 16) {
      const float2 v = real ? load2_coherent(sr, 8 * (s * d.G + sh_h)) : make_float2(-INFINITY, 0.0f);
      f_sh[s * Gp + sh_h] = v.y > 0.0f ? __builtin_amdgcn_exp2f(v.x - m) * rz : 0.0f;
    }
  }
  __syncthreads();
}

// Pooling and both stages for pair p, run by the pair's last score
// workgroup once every split has published (so the chunk weights and split
// statistics are read with device-coherent loads); the splits cover every
// complete chunk. L is the pair's sequence length (after this step's append).
__device__ __forceinline__ void pool_select(const Dims &d, const nosa_state &st, int L_in,
                                            const float *ws_e, const float *ws_stats,
                                            int c_pad, int n_splits, int32_t *sel,
                                            int32_t *n_sel, uint8_t *kind_out, float *dbg,
                                            int p) {
  const int Gp = padded_group(d.G);
  extern __shared__ __align__(16) uint8_t smem[];
  float *f_sh = reinterpret_cast<float *>(smem);                            // [n_splits][Gp]
  float *a_sh = f_sh + n_splits * Gp;                                       // [c_pad]
  uint32_t *el_sh = reinterpret_cast<uint32_t *>(a_sh + c_pad);             // [elig_words]
  uint8_t *kind = reinterpret_cast<uint8_t *>(el_sh + d.elig_words);        // [NB_max]
  __shared__ TopkLds tk;

  const int t = threadIdx.x;

  const int L = max(0, min(L_in, d.max_context));
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
  const int sh_h = t >> 4, sh_j = t & 15;
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(ws_stats + (size_t)2 * p * n_splits * d.G, (uint32_t)n_splits * d.G * 8);
  // thread (sh_h, sh_j): head sh_h's statistics of splits sh_j + 16 i
  float2 stv_raw[kStatBatches];
#pragma unroll
  for (int i = 0; i < kStatBatches; ++i) {
    const int s = sh_j + 16 * i;
    stv_raw[i] = (sh_h < d.G && s < n_splits) ? load2_coherent(sr, 8 * (s * d.G + sh_h))
                                              : make_float2(-INFINITY, 0.0f);
  }
  // 0. issue the global loads together, so the kernel waits for one memory
  // round trip: the first batch of chunk weights (coalesced float4s of the
  // chunk-major [c][Gp] array, bounded by the buffer's extent), the split
  // statistics (above), the candidates' agnostic scores, eligibility
  const int n4_ext = c_pad * Gp / 4;
  const __amdgpu_buffer_rsrc_t er = make_rsrc(ws_e + (size_t)p * c_pad * Gp, (uint32_t)n4_ext * 16);
  float4 eb[kLoadBatch];
#pragma unroll
  for (int u = 0; u < kLoadBatch; ++u) {
    const int k4 = t + kTopkThreads * u;
    eb[u] = k4 < n4_ext ? load4_coherent(er, 16 * k4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float *be = st.blk_e + (size_t)p * d.NB_max;
  const float e0_raw = d.n_sink + t < d.NB_max ? get(&be[d.n_sink + t]) : 0.0f;
  const int n4 = do_q ? C * Gp / 4 : 0;
  const bool have0 = t < n_cand;
  const float e0 = (do_e && have0) ? e0_raw : 0.0f;
  for (int i = t; i < d.elig_words; i += kTopkThreads)
    el_sh[i] = st.eligible[(size_t)p * d.elig_words + i];
  for (int bb = t; bb < nb; bb += kTopkThreads)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);
  topk_lds_init(tk);

  NOSA_PHASE(p, kPhasePoolRow, 4);
  pool_factors(d, Gp, used, do_q, sr, stv_raw, f_sh);
  NOSA_PHASE(p, kPhasePoolRow, 5);

  // 2. chunk scores a_c = sum over the group's heads of the head's softmax
  // weight, once per chunk (a chunk shared by two blocks gives both the same
  // value): each float4 covers 4 heads of one chunk, the Gp / 4 lanes of a
  // chunk are adjacent and combine with DPP lane exchanges
  if (do_q) {
    for (int k0 = 0; k0 < n4; k0 += kTopkThreads * kLoadBatch) {     // uniform
      if (k0 > 0) {
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int k4 = k0 + t + kTopkThreads * u;
          eb[u] = k4 < n4 ? load4_coherent(er, 16 * k4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      if (Gp == 4)
        chunk_scores<4>(eb, k0, n4, n_splits, f_sh, a_sh);
      else if (Gp == 8)
        chunk_scores<8>(eb, k0, n4, n_splits, f_sh, a_sh);
      else
        chunk_scores<16>(eb, k0, n4, n_splits, f_sh, a_sh);
    }
  }
  __syncthreads();
  NOSA_PHASE(p, kPhasePoolRow, 6);

  finish_select(d, st, p, nb, win_lo, n_cand, C, do_q, do_e, a_sh, el_sh, be, e0, kind, sel,
                n_sel, kind_out, dbg, tk);
}

}  // namespace
}  // namespace nosa
