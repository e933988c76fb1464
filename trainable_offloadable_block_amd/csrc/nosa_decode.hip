// Sparse decode attention over the selected blocks (NOSA-1B 核心组件揭秘,
// 解码阶段如何只用 64 个 KV 块; aiwiki "NOSA", How NOSA works: the eviction
// score enters the logits as an additive bias; l189 article, 2.1, eq. 8).
//
// decode_kernel: grid (splits, pairs), 4 waves per workgroup. Each wave
//   streams its share of the pair's selected blocks half by half (32 tokens),
//   with the next half's loads in flight while the current one is computed:
//   logits S^T = K Q^T on MFMA (the GQA group padded to 16 rows of the
//   16x16x32 shape), an online softmax in the log2 domain with the bias
//   fused, and O^T += V^T P^T on MFMA with P split into bf16 hi + lo parts
//   (P alone in bf16 would cost ~1e-3 relative error). The 4 waves merge in
//   LDS into one partial (m, l, o) per split; the last workgroup of a pair to
//   finish merges all splits and writes the normalised output (a pair with a
//   single split writes it straight from the LDS merge). A pair's workgroups
//   are placed on one XCD (grid_unit).
#include <hip/hip_ext.h>

#include <mutex>

#include "nosa_internal.h"
#include "nosa_lanes.h"
#include "nosa_phase.h"

// Scratch of nosa_sparse_decode_static, for callers that cannot allocate: the
// decode workspace (per-pair arrival counters at offset 0, then the split
// partials) of every call on a GPU lives here. Each GPU the library runs on
// holds its own copy until the process ends. Host code never uses this name
// as an address: it takes the copy's device address from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[nosa::kDecodeStaticScratchBytes];

namespace nosa {
namespace {

#ifndef NOSA_DECODE_MIN_WAVES
#define NOSA_DECODE_MIN_WAVES 2     // <= 256 registers: two workgroups per CU fit
#endif

#ifndef NOSA_DECODE_WAVES
#define NOSA_DECODE_WAVES 4         // waves per workgroup (one workgroup per CU at 16K)
#endif
constexpr int kDecWaves = NOSA_DECODE_WAVES;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kMaxSplits = 32;   // k <= 128 blocks, >= 4 blocks per split
constexpr float kLog2e = 1.4426950408889634f;

// A-row r of tile t <-> row 8*(r/4) + 4*t + (r%4) of a 32-row group, so that
// lane group j ends up holding rows 8j .. 8j+7 of the group (see select).
__device__ inline int tile_row(int r, int t) { return 8 * (r >> 2) + 4 * t + (r & 3); }

__device__ inline uint4 ldg16(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor over [base, base + bytes): loads past the end read 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The KV stream is read once per step: non-temporal loads (cache policy
// nt), which stream from HBM markedly faster than loads that allocate in the
// caches.
constexpr int kStream = 2;
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream));
}

// Bytes past a sequence's length inside its newest block are zero (append
// clears a block when a token opens it, prefill clears the tail of the last
// partial block), so V there is finite and its probability 0 keeps it out.

// One 32-token half of a selected block, as this lane's MFMA operands.
struct Half {
  uint4 k[2][4];   // K rows of the two QK tiles, 4 k-steps each
  uint4 v[8];      // the half's 8 V tiles: 8 keys of one dim per lane
  float4 s[2];     // eviction scores of this lane's 8 keys: 8 (lane / 16) .. + 7
  int key_base;    // token index of the half's first key (wave-uniform)
  int ok;          // 0: past the wave's list or an invalid entry (uniform)
};

struct DecodeArgs {
  const int32_t *sel, *phys;
  __amdgpu_buffer_rsrc_t kv;   // this pair's blocks
  __amdgpu_buffer_rsrc_t ts;   // this pair's eviction scores
  int koff[2], voff, soff;     // per-lane byte offsets inside a block / half / scores
  int p, slots, e_first, e_end;
};

// Issues the loads of half j (< the wave's half count) of the wave's list
// (entries e_first, e_first + 4, ...; two halves each). Lane i holds the
// block and slot ids of the wave's i-th entry (loaded once at the start), so
// no memory round trip precedes the loads. The loads are unconditional and
// their offsets wave-uniform (no branch defines them), so the compiler keeps
// one half in flight while another is computed; an invalid entry reads slot
// 0, is marked not ok and sets `bad`.
__device__ inline void load_half(Half &hb, int j, const DecodeArgs &a, const Dims &d,
                                 int lane_blk, int lane_slot, bool &bad) {
  const int half = j & 1;
  int blk = __builtin_amdgcn_readlane(lane_blk, j >> 1);
  int slot = __builtin_amdgcn_readlane(lane_slot, j >> 1);
  const bool ok = blk >= 0 && blk < d.NB_max && slot >= 0 && slot < a.slots;
  hb.ok = ok ? 1 : 0;
  bad = bad || !ok;
  blk = __builtin_amdgcn_readfirstlane(ok ? blk : 0);
  slot = __builtin_amdgcn_readfirstlane(ok ? slot : 0);
  const int kbase = slot * (kBlockElems * 2) + half * (32 * kHeadDim * 2);
  const int vbase = slot * (kBlockElems * 2) + kBlock * kHeadDim * 2 + half * 8192;
  hb.key_base = blk * kBlock + 32 * half;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) hb.k[t][s] = bload16(a.kv, a.koff[t] + 64 * s, kbase);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) hb.v[dt] = bload16(a.kv, a.voff + 1024 * dt, vbase);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    hb.s[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                             a.ts, a.soff + 16 * i, hb.key_base * 4, kStream));
}

// Online-softmax update with one half: logits on MFMA, then O^T += V^T P^T.
__device__ inline void process_half(Half &hb, const bf16x8 (&qop)[4], float qscale,
                                    float bscale, int L, int lg, float &m_run, float &l_run,
                                    f32x4 (&o)[8]) {
  if (!hb.ok) return;                          // wave-uniform
  f32x4 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t] = mfma16x16x32(as_bf16x8(hb.k[t][s]), qop[s], acc[t]);
  }
  const int key0 = hb.key_base + 8 * lg;       // this lane's first key
  float x[8];
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float sv = hb.s[m >> 2][m & 3];
    const float lg2 = acc[m >> 2][m & 3] * qscale + sv * bscale;
    x[m] = (key0 + m) < L ? lg2 : -INFINITY;
    mx = fmaxf(mx, x[m]);
  }
  mx = xor32_max(xor16_max(mx));
  const float m_new = fmaxf(m_run, mx);
  if (m_new == -INFINITY) return;              // wave-uniform: nothing valid
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);    // 0 while m_run = -inf
  m_run = m_new;
  float psum = 0.0f;
  uint32_t phi[4], plo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 pm = {__builtin_amdgcn_exp2f(x[2 * i] - m_new), __builtin_amdgcn_exp2f(x[2 * i + 1] - m_new)};
    psum += pm[0] + pm[1];
    // P = hi + lo, both bf16 (round to nearest even)
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(pm, bf16x2));
    const f32x2 back = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u)};
    phi[i] = hi;
    plo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pm - back, bf16x2));
  }
  l_run = l_run * alpha + psum;
  const bf16x8 bhi = __builtin_bit_cast(bf16x8, uint4{phi[0], phi[1], phi[2], phi[3]});
  const bf16x8 blo = __builtin_bit_cast(bf16x8, uint4{plo[0], plo[1], plo[2], plo[3]});
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    o[dt] *= alpha;
    o[dt] = mfma16x16x32(as_bf16x8(hb.v[dt]), bhi, o[dt]);
    o[dt] = mfma16x16x32(as_bf16x8(hb.v[dt]), blo, o[dt]);
  }
}

__device__ inline float load_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Final merge of a pair's split partials, by the pair's last workgroup.
// Thread t owns outputs t + 256 i (i < NI; NI * 256 >= G * 128). Every
// partial is read with device-coherent loads, SB = 16 / NI splits per batch,
// the first batch issued before the (m, l) round trip so the two overlap.
template <int NI>
__device__ void merge_splits(const Dims &d, int p, int b, int g, int n_splits,
                             const float *mlf, const float *ws_o, float *sm, float *out) {
  constexpr int SB = 16 / NI;
  const int t = threadIdx.x;
  const int n_out = d.G * kHeadDim;
  const float *mlp = mlf + (size_t)2 * p * n_splits * d.G;
  const float *op = ws_o + (size_t)p * n_splits * n_out;
  float *sm_w = sm;                                   // [kMaxSplits][16]: m, then weights
  float *sm_lv = sm_w + kMaxSplits * 16;              // [kMaxSplits][16]: l
  float *sm_lh = sm_lv + kMaxSplits * 16;             // [16]: merged l
  float v[SB][NI];
  auto issue = [&](int sp0) {
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int idx = t + kDecThreads * i;
        v[u][i] = (sp0 + u < n_splits && idx < n_out)
                      ? load_agent(&op[(size_t)(sp0 + u) * n_out + idx]) : 0.0f;
      }
  };
  issue(0);
  for (int i = t; i < n_splits * d.G; i += kDecThreads) {
    sm_w[i] = load_agent(&mlp[2 * i]);
    sm_lv[i] = load_agent(&mlp[2 * i + 1]);
  }
  __syncthreads();
  if (t < d.G) {
    float M = -INFINITY;
    for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, sm_w[sp * d.G + t]);
    float lsum = 0.0f;
    for (int sp = 0; sp < n_splits; ++sp) {
      const float f = M == -INFINITY ? 0.0f : exp2f(sm_w[sp * d.G + t] - M);
      sm_w[sp * d.G + t] = f;
      lsum += f * sm_lv[sp * d.G + t];
    }
    sm_lh[t] = lsum;
  }
  __syncthreads();
  float acc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] = 0.0f;
  for (int sp0 = 0; sp0 < n_splits; sp0 += SB) {
    if (sp0 > 0) issue(sp0);
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int idx = t + kDecThreads * i;
        if (sp0 + u < n_splits && idx < n_out) acc[i] += sm_w[(sp0 + u) * d.G + idx / kHeadDim] * v[u][i];
      }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = t + kDecThreads * i;
    if (idx < n_out) {
      const int hh = idx / kHeadDim, dim = idx % kHeadDim;
      const float lsum = sm_lh[hh];
      out[((size_t)b * d.Hq + g * d.G + hh) * kHeadDim + dim] = lsum > 0.0f ? acc[i] / lsum : 0.0f;
    }
  }
}

// merge_splits for a group of 4, 8 or 16 heads (NV = max(1, G / 8)): thread
// t owns the float4s of outputs 4 (t + 256 j) .. + 3 below G * 128 (one head
// each; at G = 4 the last two waves own none), read with unconditional
// 16-byte device-coherent buffer loads (a split past n_splits reads zeros),
// SB splits per batch: every batch is one memory round trip, so SB covers
// the pair's splits in one batch up to 16 / NV of them.
constexpr int kAgentCoherent = 16;   // buffer cache policy: sc1 (device scope)

template <int NV, int SB>
__device__ void merge_splits_v(const Dims &d, int p, int b, int g, int n_splits,
                               const float *mlf, const float *ws_o, float *sm, float *out) {
  const int t = threadIdx.x;
  const int n_out = d.G * kHeadDim;                   // 512, 1024 or 2048
  const float *mlp = mlf + (size_t)2 * p * n_splits * d.G;
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(ws_o + (size_t)p * n_splits * n_out, (uint32_t)(n_splits * n_out * 4));
  float4 v[SB][NV];
  auto issue = [&](int sp0) {
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < NV; ++j)
        v[u][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ro, ((sp0 + u) * n_out + 4 * (t + kDecThreads * j)) * 4,
                                                 0, kAgentCoherent));
  };
  issue(0);
  // split statistics without LDS or barriers: for its j-th float4 a lane's
  // head is 2 w + 8 j (lanes 0..31) or 2 w + 8 j + 1 (lanes 32..63); lane
  // (32 half + sp) loads that head's (m, l) of split sp, the two halves
  // reduce separately, and each lane reads its half's weights back by lane
  const int lane = t & 63, half = lane >> 5, spl = lane & 31;
  const int w = t >> 6;
  float fw[NV], lsum[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int hh = 2 * w + (kDecThreads / 32) * j + half;
    float m = -INFINITY, lv = 0.0f;
    if (spl < n_splits && hh < d.G) {
      m = load_agent(&mlp[2 * (spl * d.G + hh)]);
      lv = load_agent(&mlp[2 * (spl * d.G + hh) + 1]);
    }
    const float M = xor16_max(row16_max(m));         // over the lane's half
    const float f = (m == -INFINITY) ? 0.0f : exp2f(m - M);
    fw[j] = f;
    lsum[j] = xor16_sum(row16_sum(f * lv));
  }
  float4 acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp0 = 0; sp0 < n_splits; sp0 += SB) {
    if (sp0 > 0) issue(sp0);
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (sp0 + u < n_splits) {                       // uniform
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const float wa = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fw[j]), sp0 + u));
          const float wb = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fw[j]), 32 + sp0 + u));
          const float wgt = half ? wb : wa;
          acc[j].x += wgt * v[u][j].x;
          acc[j].y += wgt * v[u][j].y;
          acc[j].z += wgt * v[u][j].z;
          acc[j].w += wgt * v[u][j].w;
        }
      }
  }
  float *ob = out + ((size_t)b * d.Hq + g * d.G) * kHeadDim;   // the group's heads, contiguous
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int idx = 4 * (t + kDecThreads * j);
    if (idx >= n_out) break;                          // wave-uniform (G = 4)
    const float ls = lsum[j];
    *reinterpret_cast<float4 *>(ob + idx) =
        ls > 0.0f ? make_float4(acc[j].x / ls, acc[j].y / ls, acc[j].z / ls, acc[j].w / ls)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__global__ __launch_bounds__(kDecThreads, NOSA_DECODE_MIN_WAVES) void decode_kernel(
    Dims d, const int32_t *__restrict__ seq_len, const uint16_t *__restrict__ q,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ phys,
    const int32_t *__restrict__ n_sel, const uint16_t *__restrict__ kv, int slots_per_pair,
    const float *__restrict__ tok_s, float *__restrict__ ws_o, float2 *__restrict__ ws_ml,
    int32_t *__restrict__ ws_count, int bps, int n_splits, float *__restrict__ out,
    uint32_t *status) {
  int split, p;
  grid_unit(split, p);
  NOSA_PHASE(p, split, 0);
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int h = l & 15, lg = l >> 4;
  // lane i: block and slot ids of this wave's i-th list entry, loaded
  // before the list length is known (every entry < k exists), so the first
  // KV loads wait for one memory round trip, not two
  const int e_lane = split * bps + w + kDecWaves * l;
  int lane_blk = -1, lane_slot = -1;
  if (l < 16 && e_lane < d.k) {
    lane_blk = sel[(size_t)p * d.k + e_lane];
    lane_slot = phys[(size_t)p * d.k + e_lane];
  }
  const int L = seq_len[b];
  const int ns = max(0, min(n_sel[p], d.k));
  // wait for the ids here, on every path: a path that skipped the wait
  // would leave the compiler waiting for every load in flight at each
  // iteration of the streaming loop, the prefetched half included
  asm volatile("" ::"v"(lane_blk), "v"(lane_slot));

  __shared__ float sm_m[kDecWaves][16], sm_l[kDecWaves][16];
  __shared__ __align__(16) float sm_o[kDecWaves][16][kHeadDim + 4];
  auto waves_max = [&](int hh) {
    float M = sm_m[0][hh];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    return M;
  };
  __shared__ int sm_last;

  DecodeArgs a;
  a.sel = sel;
  a.phys = phys;
  a.kv = make_rsrc(kv + (size_t)p * slots_per_pair * kBlockElems,
                   (uint32_t)slots_per_pair * kBlockElems * 2);
  a.ts = make_rsrc(tok_s + (size_t)p * d.tok_stride, (uint32_t)d.tok_stride * 4);
  a.koff[0] = tile_row(h, 0) * kHeadDim * 2 + 16 * lg;
  a.koff[1] = tile_row(h, 1) * kHeadDim * 2 + 16 * lg;
  a.voff = 16 * l;   // V tile: lane l holds dim l % 16, tokens 8 (l / 16) .. + 7
  a.soff = 32 * (l >> 4);   // lane group lg reads the scores of keys 8 lg .. 8 lg + 7
  a.p = p;
  a.slots = slots_per_pair;
  a.e_first = split * bps + w;
  a.e_end = min(ns, split * bps + bps);
  const int n_mine = a.e_first < a.e_end ? (a.e_end - a.e_first + kDecWaves - 1) / kDecWaves : 0;
  // n_mine <= 16: only lanes below it hold entries of the list

  const int nh = 2 * n_mine;

  Half A, B;
  bool bad = false;                                  // wave-uniform
  if (nh > 0) load_half(A, 0, a, d, lane_blk, lane_slot, bad);

  bf16x8 qop[4];
  if (h < d.G) {
    const uint16_t *qh = q + ((size_t)b * d.Hq + g * d.G + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(ldg16(qh + 32 * s));
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  const float qscale = 0.08838834764831845f * kLog2e;   // log2(e) / sqrt(128)
  const float bscale = d.bias ? kLog2e : 0.0f;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // nh is even (two halves per entry); the last pair is peeled so that no
  // load inside the loop is conditional
  for (int j = 0; j < nh - 2; j += 2) {
    load_half(B, j + 1, a, d, lane_blk, lane_slot, bad);
    process_half(A, qop, qscale, bscale, L, lg, m_run, l_run, o);
    load_half(A, j + 2, a, d, lane_blk, lane_slot, bad);
    process_half(B, qop, qscale, bscale, L, lg, m_run, l_run, o);
  }
  if (nh > 0) {
    load_half(B, nh - 1, a, d, lane_blk, lane_slot, bad);
    process_half(A, qop, qscale, bscale, L, lg, m_run, l_run, o);
    process_half(B, qop, qscale, bscale, L, lg, m_run, l_run, o);
  }

  NOSA_PHASE_WAVE(p, split, 6 + w);
  if (bad && l == 0) atomicOr(status, NOSA_STATUS_BAD_SEL);
  // lane (h, lg): head h's running max, its keys' partial sum, and
  // O^T[16*dt + 4*lg + i][h]; merge the 4 waves in LDS
  l_run = xor32_sum(xor16_sum(l_run));
  if (lg == 0) {
    sm_m[w][h] = m_run;
    sm_l[w][h] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][h][16 * dt + 4 * lg + i] = o[dt][i];
  __syncthreads();
  NOSA_PHASE(p, split, 2);
  if (n_splits == 1 && (d.G == 4 || d.G == 8 || d.G == 16)) {   // uniform
    // the pair's only split: normalise and write, a float4 (one head) each
    float *ob = out + ((size_t)b * d.Hq + g * d.G) * kHeadDim;
    for (int j = 0; 4 * (threadIdx.x + kDecThreads * j) < d.G * kHeadDim; ++j) {
      const int idx = 4 * (threadIdx.x + kDecThreads * j);
      const int hh = idx / kHeadDim, dim = idx % kHeadDim;
      const float M = waves_max(hh);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      float lsum = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
          const float f = exp2f(sm_m[ww][hh] - M);
          const float4 ov = *reinterpret_cast<const float4 *>(&sm_o[ww][hh][dim]);
          acc.x += f * ov.x;
          acc.y += f * ov.y;
          acc.z += f * ov.z;
          acc.w += f * ov.w;
          lsum += f * sm_l[ww][hh];
        }
      }
      *reinterpret_cast<float4 *>(ob + idx) =
          lsum > 0.0f ? make_float4(acc.x / lsum, acc.y / lsum, acc.z / lsum, acc.w / lsum)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  if (n_splits == 1) {                         // uniform: the pair's only split
    for (int idx = threadIdx.x; idx < d.G * kHeadDim; idx += kDecThreads) {
      const int hh = idx / kHeadDim, dim = idx % kHeadDim;
      const float M = waves_max(hh);
      float acc = 0.0f, lsum = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
          const float f = exp2f(sm_m[ww][hh] - M);
          acc += f * sm_o[ww][hh][dim];
          lsum += f * sm_l[ww][hh];
        }
      }
      out[((size_t)b * d.Hq + g * d.G + hh) * kHeadDim + dim] = lsum > 0.0f ? acc / lsum : 0.0f;
    }
    return;
  }
  // publish this split's partial with device-coherent (agent-scope) stores,
  // wait for them, then count arrivals; the last workgroup of the pair reads
  // every partial back with device-coherent loads and merges. No
  // device-scope fence: that would write back the XCD's whole L2.
  const size_t part = (size_t)p * n_splits + split;
  float *mlf = reinterpret_cast<float *>(ws_ml);
  if (d.G == 4 || d.G == 8 || d.G == 16) {     // uniform: 16-byte stores, one head each
    const int n_out = d.G * kHeadDim;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(ws_o + part * n_out, (uint32_t)n_out * 4);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mlf + 2 * part * d.G, (uint32_t)d.G * 8);
    for (int j = 0; 4 * (threadIdx.x + kDecThreads * j) < n_out; ++j) {   // wave-uniform
      const int idx = 4 * (threadIdx.x + kDecThreads * j);
      const int hh = idx / kHeadDim, dim = idx % kHeadDim;
      const float M = waves_max(hh);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      float lsum = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
          const float f = exp2f(sm_m[ww][hh] - M);
          const float4 ov = *reinterpret_cast<const float4 *>(&sm_o[ww][hh][dim]);
          acc.x += f * ov.x;
          acc.y += f * ov.y;
          acc.z += f * ov.z;
          acc.w += f * ov.w;
          lsum += f * sm_l[ww][hh];
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro, idx * 4, 0,
                                             kAgentCoherent);
      if (dim == 0)
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u32x2, make_float2(M, lsum)), rm, hh * 8, 0, kAgentCoherent);
    }
  } else {
  for (int idx = threadIdx.x; idx < d.G * kHeadDim; idx += kDecThreads) {
    const int hh = idx / kHeadDim, dim = idx % kHeadDim;
    const float M = waves_max(hh);
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) {
        const float f = exp2f(sm_m[ww][hh] - M);
        acc += f * sm_o[ww][hh][dim];
        lsum += f * sm_l[ww][hh];
      }
    }
    __hip_atomic_store(&ws_o[(part * d.G + hh) * kHeadDim + dim], acc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (dim == 0) {
      __hip_atomic_store(&mlf[2 * (part * d.G + hh)], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&mlf[2 * (part * d.G + hh) + 1], lsum, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  }
  __builtin_amdgcn_s_waitcnt(0);          // this thread's stores have landed
  __syncthreads();
  NOSA_PHASE(p, split, 3);
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(&ws_count[p], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              n_splits - 1;
  __syncthreads();
  NOSA_PHASE(p, split, 4);
  if (!sm_last) return;
  constexpr int NV16 = (16 * 32 + kDecThreads - 1) / kDecThreads;   // 2
  if ((d.G == 4 || d.G == 8) && n_splits <= 4)
    merge_splits_v<1, 4>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  else if (d.G == 4 || d.G == 8)
    merge_splits_v<1, 16>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  else if (d.G == 16 && n_splits <= 4 / NV16)
    merge_splits_v<NV16, 4 / NV16>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  else if (d.G == 16)
    merge_splits_v<NV16, 16 / NV16>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  else if (d.G <= 8)
    merge_splits<4>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  else
    merge_splits<8>(d, p, b, g, n_splits, mlf, ws_o, &sm_o[0][0][0], out);
  if (threadIdx.x == 0) __hip_atomic_store(&ws_count[p], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  NOSA_PHASE(p, split, 5);
}

}  // namespace

// Zeroes n32 words (the arrival counters of a static-scratch call).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *__restrict__ w, int n32) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n32) w[i] = 0u;
}

// Per device: the scratch copy's address, and how many leading bytes of it
// are known to be zero (the counter region of the last call: a call leaves
// its counters at zero and its partials after them).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
size_t g_scratch_zero[kMaxDevices];

DecodeLayout decode_layout(const Dims &d) {
  DecodeLayout lay;
  // one round of workgroups that covers the chip: about 256 / pairs splits
  // per pair (at most kMaxSplits), each a run of bps >= 4 list entries
  // (256 workgroups of 16 blocks each at 64 pairs and k = 64)
  const int want = max(1, min(kMaxSplits, (256 + d.P - 1) / d.P));
  // (the last workgroup reads all of a pair's partials in one batch of
  // loads, so more splits cost the merge little: 32 pairs x 96 blocks at
  // GQA 16, 8 KiB partials, ran 24.5 us in runs of 12, 24.8 us in runs of
  // 16, 28.4 and 31.3 us in runs of 8 and 10, which overfill the chip)
  int bps = max(4, (d.k + want - 1) / want);
  if (const int v = tuning(NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT)) bps = v;
  while (bps < 64 && (d.k + bps - 1) / bps > kMaxSplits) bps *= 2;   // merge bound
  lay.blocks_per_split = bps;
  lay.n_splits = (d.k + bps - 1) / bps;
  const size_t parts = (size_t)d.P * lay.n_splits * d.G;
  lay.count_off = 0;
  lay.o_off = (((size_t)d.P * sizeof(int32_t) + 255) & ~(size_t)255);
  lay.ml_off = lay.o_off + ((parts * kHeadDim * sizeof(float) + 255) & ~(size_t)255);
  lay.bytes = lay.ml_off + ((parts * sizeof(float2) + 255) & ~(size_t)255);
  return lay;
}

hipError_t launch_decode(const Dims &d, const nosa_state &st, const uint16_t *q,
                         const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                         float *out, void *ws, const DecodeLayout &lay, hipStream_t s,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  char *base = static_cast<char *>(ws);
  float *ws_o = reinterpret_cast<float *>(base + lay.o_off);
  float2 *ws_ml = reinterpret_cast<float2 *>(base + lay.ml_off);
  int32_t *ws_count = reinterpret_cast<int32_t *>(base + lay.count_off);
  const int slots = d.offload ? d.k + 1 : d.NB_kv;
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(decode_kernel, dim3(lay.n_splits, d.P), dim3(kDecThreads), 0, s,
                          ev_start, ev_stop, 0, d, st.seq_len, q, sel, phys, n_sel, st.kv_dev,
                          slots, st.tok_s, ws_o, ws_ml, ws_count, lay.blocks_per_split,
                          lay.n_splits, out, st.status);
  } else {
    decode_kernel<<<dim3(lay.n_splits, d.P), kDecThreads, 0, s>>>(
        d, st.seq_len, q, sel, phys, n_sel, st.kv_dev, slots, st.tok_s, ws_o, ws_ml, ws_count,
        lay.blocks_per_split, lay.n_splits, out, st.status);
  }
  return hipGetLastError();
}

hipError_t launch_decode_static(const Dims &d, const nosa_state &st, const uint16_t *q,
                                const int32_t *sel, const int32_t *phys, const int32_t *n_sel,
                                float *out, const DecodeLayout &lay, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *ptr = nullptr;
  size_t zero_before = 0;
  const size_t counters = lay.o_off;          // counter region, a multiple of 256 bytes
  {
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {                // first call on this device (it is current)
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return e;
      }
      g_scratch_zero[dev] = 0;
    }
    ptr = g_scratch_ptr[dev];
    zero_before = g_scratch_zero[dev];
    g_scratch_zero[dev] = counters;
  }
  if (counters > zero_before) {               // counters over bytes a larger call's partials used
    const int n32 = static_cast<int>((counters - zero_before) / 4);
    zero_words_kernel<<<dim3((n32 + 255) / 256), 256, 0, s>>>(
        reinterpret_cast<uint32_t *>(static_cast<char *>(ptr) + zero_before), n32);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_decode(d, st, q, sel, phys, n_sel, out, ptr, lay, s);
}

}  // namespace nosa

#ifdef NOSA_PHASE_CLOCKS
NOSA_PHASE_READER(nosa_phase_clocks_decode)
#endif
