// Block scores of many prompt queries at once: the selection side of NOSA_S's
// sparse prefill (aiwiki "NOSA", Results: NOSA_S is sparse in both phases),
// each query scored as a decode step at its own length would score it
// (NOSA-1B 核心组件揭秘, 核心组件三): per head, a softmax over the chunks
// complete at the query's length of q . ckey / sqrt(128); summed over the
// GQA group; max-pooled over the chunks overlapping each candidate block.
//
// prefill_block_scores_kernel: grid (query groups, pairs), 8 waves. Rows of
// the MFMA tiles are (query, head) with the group padded to Gp = 4, 8 or 16
// rows per query; columns are 16 compressed keys. Each wave holds two row
// tiles (their A operands stay in registers; two workgroups share a CU); the workgroup stages the
// compressed keys in LDS 128 chunks at a time (the next 128 loaded into
// registers while the current ones are used), so every key is read from L2
// once per sweep per 16 row tiles. Two sweeps over the chunks, in the log2
// domain: an online max and sum per lane (a lane sees every 16th chunk; the
// 16 lanes of a row combine once at the end), then the normalised weights,
// their sum over the group's rows and a max over each block's chunks (the
// chunk before a tile is carried over).
#include "nosa_internal.h"
#include "nosa_lanes.h"

namespace nosa {
namespace {

constexpr int kPsWaves = 8;
constexpr int kPsRowTiles = 2;            // row tiles per wave
constexpr int kPsStage = 128;             // chunks staged in LDS at a time
constexpr int kPsPitch = kHeadDim + 8;    // LDS row pitch (elements): no bank conflicts
constexpr float kScale2 = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)

__host__ __device__ inline int padded_rows(int G) { return G <= 4 ? 4 : (G <= 8 ? 8 : 16); }
__host__ __device__ inline int queries_per_wg(int G) {
  return kPsWaves * kPsRowTiles * (16 / padded_rows(G));
}


__global__ __launch_bounds__(kPsWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void prefill_block_scores_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ q, int T, int pos0, int nb_out,
    float *__restrict__ out) {
  constexpr int NT = kPsWaves * 64;
  constexpr int kStageVecs = kPsStage * kHeadDim / 8;    // uint4 per stage
  __shared__ __align__(16) uint16_t ks_sh[kPsStage * kPsPitch];
  const int p = blockIdx.y, b = p / d.Hkv, g = p % d.Hkv;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l & 15, lg = l >> 4;
  const int Gp = padded_rows(d.G), QT = 16 / Gp;        // queries per row tile
  const int q_wg = blockIdx.x * queries_per_wg(d.G);
  const int qbase = q_wg + w * kPsRowTiles * QT;
  if (pos0 + T > st.seq_len[b]) {                        // uniform
    if (t == 0 && blockIdx.x == 0) atomicOr(st.status, NOSA_STATUS_SHORT_CONTEXT);
    return;
  }
  // lane rows: row r = 4 lg + i of tile rt is query row_q(rt, i), head
  // row_h(i); Gp >= 4, so the four rows of a lane group share one query
  auto row_q = [&](int rt) { return qbase + rt * QT + (4 * lg) / Gp; };
  auto row_h = [&](int i) { return (4 * lg + i) % Gp; };
  auto row_C = [&](int rt) {
    const int qi = row_q(rt);
    return qi < T ? min(chunks_for(pos0 + qi + 1), d.C_max) : 0;
  };
  bf16x8 a[kPsRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kPsRowTiles; ++rt) {
    // A operand: row lr of the tile, dims 32 ks + 8 lg .. + 7
    const int qa = qbase + rt * QT + lr / Gp, ha = lr % Gp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qa < T && ha < d.G)
        v = *reinterpret_cast<const uint4 *>(
            q + (((size_t)b * T + qa) * d.Hq + g * d.G + ha) * kHeadDim + 32 * ks + 8 * lg);
      a[rt][ks] = as_bf16x8(v);
    }
  }
  // chunks any query of the workgroup sees (the last query sees the most)
  const int q_last = min(q_wg + queries_per_wg(d.G), T) - 1;
  const int c_wg = q_last >= q_wg ? min(chunks_for(pos0 + q_last + 1), d.C_max) : 0;
  // chunks every query of the workgroup sees: tiles below need no causal mask
  const int c_lo = min(chunks_for(pos0 + q_wg + 1), d.C_max);
  const int n_stage = (c_wg + kPsStage - 1) / kPsStage;
  const uint4 *ck4 = reinterpret_cast<const uint4 *>(st.ckey + (size_t)p * d.C_max * kHeadDim);

  uint4 pre[kStageVecs / NT];
  auto fetch = [&](int sg) {
#pragma unroll
    for (int j = 0; j < kStageVecs / NT; ++j) {
      const int v = t + NT * j;                       // chunk v / 16, dims 8 (v % 16)
      const int c = sg * kPsStage + (v >> 4);
      pre[j] = c < c_wg ? ck4[(size_t)c * (kHeadDim / 8) + (v & 15)] : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < kStageVecs / NT; ++j) {
      const int v = t + NT * j;
      *reinterpret_cast<uint4 *>(&ks_sh[(v >> 4) * kPsPitch + 8 * (v & 15)]) = pre[j];
    }
  };
  auto tile_logits = [&](int cl, f32x4 (&acc)[kPsRowTiles]) {   // chunk tile at local chunk cl
    bf16x8 bop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bop[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(&ks_sh[(cl + lr) * kPsPitch + 32 * ks + 8 * lg]));
#pragma unroll
    for (int rt = 0; rt < kPsRowTiles; ++rt) {
      acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[rt] = mfma16x16x32(a[rt][ks], bop[ks], acc[rt]);
    }
  };

  // sweep 1: online max and sum per lane and row. The running max starts
  // at a finite floor far below any logit, so no step meets inf - inf; rows
  // that never see a chunk keep z = 0. (Separate max and sum sweeps save
  // vector work but measured slower: the extra sweep's MFMA, LDS reads and
  // barriers cost more.)
  // One exponential per logit: exp2(-|x - m|) is the factor of whichever of
  // the running sum and the new term is not at the new maximum (the other's
  // factor is 1), the same values the two-exponential form gives.
  auto online_step = [](float &m, float &z, float x) {
    const float dl = x - m;
    const float e = __builtin_amdgcn_exp2f(-fabsf(dl));
    z = dl > 0.0f ? fmaf(z, e, 1.0f) : z + e;
    m = fmaxf(m, x);
  };
  constexpr float kFloor = -1.0e30f;
  float m[kPsRowTiles][4], z[kPsRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kPsRowTiles; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[rt][i] = kFloor;
      z[rt][i] = 0.0f;
    }
  if (n_stage > 0) fetch(0);
  for (int sg = 0; sg < n_stage; ++sg) {                 // uniform
    __syncthreads();                                     // previous stage consumed
    stage();
    __syncthreads();
    if (sg + 1 < n_stage) fetch(sg + 1);
    const int n_tiles = min(kPsStage, c_wg - sg * kPsStage + 15) / 16;
    for (int tl = 0; tl < n_tiles; ++tl) {
      f32x4 acc[kPsRowTiles];
      tile_logits(16 * tl, acc);
      const int c0 = sg * kPsStage + 16 * tl, c = c0 + lr;
      if (c0 + 16 <= c_lo) {                             // uniform: every row sees the tile
#pragma unroll
        for (int rt = 0; rt < kPsRowTiles; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            online_step(m[rt][i], z[rt][i], acc[rt][i] * kScale2);
          }
      } else {
#pragma unroll
        for (int rt = 0; rt < kPsRowTiles; ++rt) {
          if (c >= row_C(rt)) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            online_step(m[rt][i], z[rt][i], acc[rt][i] * kScale2);
          }
        }
      }
    }
  }
  // combine the 16 lanes of each row
#pragma unroll
  for (int rt = 0; rt < kPsRowTiles; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mm = m[rt][i];
      mm = row16_max(mm);
      float zz = z[rt][i] * __builtin_amdgcn_exp2f(m[rt][i] - mm);
      zz = row16_sum(zz);
      m[rt][i] = mm;
      // now 1 / Z; 0 for padding heads and absent queries, whose rows the
      // unmasked tiles below still compute
      const bool real = row_h(i) < d.G && row_q(rt) < T;
      z[rt][i] = (real && zz > 0.0f) ? 1.0f / zz : 0.0f;
    }

  // sweep 2: weights, group sum, block maxima
  float carry[kPsRowTiles];                              // a of chunk 16 ct - 1
#pragma unroll
  for (int rt = 0; rt < kPsRowTiles; ++rt) carry[rt] = -INFINITY;
  if (n_stage > 0) fetch(0);
  for (int sg = 0; sg < n_stage; ++sg) {
    __syncthreads();
    stage();
    __syncthreads();
    if (sg + 1 < n_stage) fetch(sg + 1);
    const int n_tiles = min(kPsStage, c_wg - sg * kPsStage + 15) / 16;
    for (int tl = 0; tl < n_tiles; ++tl) {
      f32x4 acc[kPsRowTiles];
      tile_logits(16 * tl, acc);
      const int ct = sg * (kPsStage / 16) + tl;
      const int c = 16 * ct + lr;
      const bool full = 16 * ct + 16 <= c_lo;            // uniform
#pragma unroll
      for (int rt = 0; rt < kPsRowTiles; ++rt) {
        float s = 0.0f;
        const bool in = full || c < row_C(rt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[rt][i], kScale2, -m[rt][i]));
          if (in) s = fmaf(e, z[rt][i], s);
        }
        // the query's other lane groups (Gp = 8: two per query; 16: four)
        if (Gp >= 8) s = xor16_sum(s);
        if (Gp >= 16) s = xor32_sum(s);
        // lane group lg holds a_c (chunk c) of query row_q(rt)
        const float prev = row_shift<-1>(s);             // chunk c - 1 (lane 0: its own)
        const float up = lr == 0 ? carry[rt] : prev;
        float y = fmaxf(s, row_shift<1>(s));
        y = fmaxf(y, row_shift<2>(s));
        y = fmaxf(y, row_shift<3>(s));
        y = fmaxf(y, up);                                // lane 4j: block 4 ct + j
        carry[rt] = __shfl(s, 15, 16);
        const int qi = row_q(rt);
        const bool writer = (lr & 3) == 0 && qi < T && (Gp < 8 || (lg & (Gp / 4 - 1)) == 0);
        const int blk = 4 * ct + (lr >> 2);
        if (writer && blk < nb_out) {
          const int L = pos0 + qi + 1;
          const int win_lo = max(d.n_sink, blocks_for(L) - d.n_win);
          const bool cand = blk >= d.n_sink && blk < win_lo;
          out[((size_t)p * T + qi) * nb_out + blk] = cand ? y : -INFINITY;
        }
      }
    }
  }
  // blocks past the swept tiles hold no candidate of these queries
  const int n_ct = (c_wg + 15) / 16;
#pragma unroll
  for (int rt = 0; rt < kPsRowTiles; ++rt)
    for (int qq = 0; qq < QT; ++qq) {
      const int qi = qbase + rt * QT + qq;
      if (qi >= T) break;
      for (int blk = 4 * n_ct + l; blk < nb_out; blk += 64)
        out[((size_t)p * T + qi) * nb_out + blk] = -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_block_scores(const Dims &d, const nosa_state &st, const uint16_t *q,
                                       int T, int pos0, float *out, hipStream_t s) {
  const int QG = queries_per_wg(d.G);
  const int nb_out = blocks_for(pos0 + T);
  prefill_block_scores_kernel<<<dim3((T + QG - 1) / QG, d.P), kPsWaves * 64, 0, s>>>(
      d, st, q, T, pos0, nb_out, out);
  return hipGetLastError();
}

}  // namespace nosa
