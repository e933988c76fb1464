// Sparse prefill in NOSA_S's style (aiwiki "NOSA", Results: sparse in both
// phases): every prompt query selects and attends as a decode step at its own
// length would, with every candidate block eligible (the never-reselect state
// begins with decoding; aiwiki "NOSA", How NOSA works).
//
// prefill_select_kernel: grid (queries, pairs), one workgroup per query:
//   stage 1 takes the k_q candidates of highest block score (from
//   nosa_prefill_block_scores), stage 2 the k_e' others of highest agnostic
//   score; the ascending list of sink, window and selected blocks. A prompt
//   of at most 512 candidate blocks per query runs one wave per workgroup
//   (up to 8 keys a lane): the work per query is a short chain of dependent
//   reductions, so more resident workgroups per CU beat wider ones.
// prefill_attend_kernel: grid (query groups, pairs), 8 waves; a wave takes
//   16 / Gp consecutive queries (16 MFMA columns of (query, head)); the
//   workgroup forms the union of its queries' selections in LDS and stages
//   each union block there once for its 8 waves (the next block loaded into
//   registers meanwhile), and each wave runs over it half by half:
//   logits S^T = K Q^T on MFMA, a column is masked where its query did not
//   select the block or the key lies past the query's position, an online
//   softmax per column in the log2 domain with the eviction-score bias, and
//   O^T += V^T P^T on MFMA (P split into bf16 hi + lo). Resident KV only.
#include "nosa_select_dev.h"

namespace nosa {
namespace {

__host__ __device__ inline int pa_rows(int G) { return G <= 4 ? 4 : (G <= 8 ? 8 : 16); }

// ---------------------------------------------------------------- select
template <int R, int NT>
__device__ __forceinline__ void pf_stages(const Dims &d, const float *__restrict__ sc,
                                          const float *__restrict__ be, int n_cand,
                                          uint8_t *kind, TopkLds &tk) {
  const int t = threadIdx.x;
  if (d.k_q > 0) {
    uint64_t kq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + NT * r, bb = d.n_sink + i;
      kq[r] = i < n_cand ? compose_key(sc[bb], bb) : 0;
    }
    wg_topk<R, NT>(kq, d.k_q, d.n_sink, kind, NOSA_KIND_QUERY, tk);
    __syncthreads();
  }
  if (d.k_e_dyn > 0) {
    uint64_t ke[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + NT * r, bb = d.n_sink + i;
      ke[r] = (i < n_cand && kind[bb] != NOSA_KIND_QUERY) ? compose_key(be[bb], bb) : 0;
    }
    wg_topk<R, NT>(ke, d.k_e_dyn, d.n_sink, kind, NOSA_KIND_AGNOSTIC, tk);
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void prefill_select_kernel(
    Dims d, nosa_state st, const float *__restrict__ scores, int T, int pos0, int nb_out,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel) {
  extern __shared__ __align__(16) uint8_t kind[];          // [NB_max]
  __shared__ TopkLds tk;
  __shared__ int cnt_sh[2][NT / 64];
  const int qi = blockIdx.x, p = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int L = pos0 + qi + 1;
  const int nb = blocks_for(L);
  const int win_lo = max(d.n_sink, nb - d.n_win);
  const int n_cand = max(0, win_lo - d.n_sink);
  for (int bb = t; bb < nb; bb += NT)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);
#pragma unroll
  for (int i = 0; i < kTopkBins / NT; ++i) {
    tk.hist[0][t + NT * i] = 0;
    tk.hist[1][t + NT * i] = 0;
  }
  __syncthreads();
  if (n_cand > 0) {                                         // uniform
    const float *sc = scores + ((size_t)p * T + qi) * nb_out;
    const float *be = st.blk_e + (size_t)p * d.NB_max;
    const int m = (n_cand + NT - 1) / NT;
    if (m <= 1) pf_stages<1, NT>(d, sc, be, n_cand, kind, tk);
    else if (m <= 2) pf_stages<2, NT>(d, sc, be, n_cand, kind, tk);
    else if (m <= 4) pf_stages<4, NT>(d, sc, be, n_cand, kind, tk);
    else if (m <= 8 || NT == 64) pf_stages<8, NT>(d, sc, be, n_cand, kind, tk);   // NT 64: n_cand <= 512
    else pf_stages<kMaxCandPerThread, NT>(d, sc, be, n_cand, kind, tk);
  }
  __syncthreads();
  // ascending list: ballot + prefix count per NT blocks
  int32_t *sp = sel + ((size_t)p * T + qi) * d.k;
  int running = 0;
  for (int base = 0; base < nb; base += NT) {      // uniform
    const int bb = base + t;
    const bool in = bb < nb && kind[bb] != NOSA_KIND_NONE;
    const uint64_t mask = __ballot(in);
    const int below = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) cnt_sh[(base / NT) & 1][w] = __popcll(mask);
    __syncthreads();
    const int *cs = cnt_sh[(base / NT) & 1];
    int off = running, tot = 0;
#pragma unroll
    for (int ww = 0; ww < NT / 64; ++ww) {
      if (ww < w) off += cs[ww];
      tot += cs[ww];
    }
    off += below;
    if (in && off < d.k) sp[off] = bb;
    running += tot;
  }
  for (int j = running + t; j < d.k; j += NT) sp[j] = -1;
  if (t == 0) n_sel[(size_t)p * T + qi] = min(running, d.k);
}

// ---------------------------------------------------------------- attend
constexpr int kPaWaves = 8;
constexpr int kPaKPitch = kHeadDim * 2 + 16;     // LDS bytes per K row: no bank conflicts
constexpr int kPaKBytes = kBlock * kPaKPitch;    // K part of a staged block
constexpr int kPaVBytes = kBlock * kHeadDim * 2; // V part (tile order, as stored)

__host__ __device__ inline int pa_queries_per_wave(int G) { return 16 / pa_rows(G); }

// A-row r of tile t <-> key 8*(r/4) + 4*t + (r%4) of a 32-key half, so that
// lane group j holds keys 8j .. 8j+7 of the half (the decode kernel's order).
__device__ inline int pa_tile_row(int r, int t) { return 8 * (r >> 2) + 4 * t + (r & 3); }

// grid (query groups, pairs), 8 waves (two workgroups share a CU, so two
// blocks are in flight per CU); dynamic LDS: the workgroup's
// selection bitmaps [queries][words] and their union [words].
__global__ __launch_bounds__(kPaWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void prefill_attend_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ q, int T, int pos0,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ n_sel,
    float *__restrict__ out) {
  constexpr int NT = kPaWaves * 64;
  constexpr int kVecs = kBlockElems * 2 / 16 / NT;           // uint4 per thread per block
  __shared__ __align__(16) uint8_t kv_sh[kPaKBytes + kPaVBytes];
  __shared__ float s_sh[kBlock];
  extern __shared__ uint32_t dyn[];
  const int p = blockIdx.y, b = p / d.Hkv, g = p % d.Hkv;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, h = l & 15, lg = l >> 4;
  const int Gp = pa_rows(d.G), QT = pa_queries_per_wave(d.G), QW = kPaWaves * QT;
  const int words = d.elig_words;
  uint32_t *bits = dyn;                                      // [QW][words]
  uint32_t *orb = dyn + QW * words;                          // [words]
  const int qw0 = blockIdx.x * QW;                           // first query of the workgroup

  // 1. selection bitmaps of the workgroup's queries, and their union
  for (int i = t; i < (QW + 1) * words; i += NT) dyn[i] = 0u;
  __syncthreads();
  bool bad = false;
  for (int ql = w; ql < QW; ql += kPaWaves) {
    const int qi = qw0 + ql;
    if (qi >= T) break;
    const int ns = max(0, min(n_sel[(size_t)p * T + qi], d.k));
    for (int e = l; e < ns; e += 64) {
      const int blk = sel[((size_t)p * T + qi) * d.k + e];
      if (blk >= 0 && blk < d.NB_max && blk * kBlock <= pos0 + qi) {
        atomicOr(&bits[ql * words + (blk >> 5)], 1u << (blk & 31));
        atomicOr(&orb[blk >> 5], 1u << (blk & 31));
      } else {
        bad = true;
      }
    }
  }
  __syncthreads();

  // 2. this lane's column: query ql = w * QT + h / Gp, head hh = h % Gp
  const int ql = w * QT + h / Gp, hh = h % Gp, qi = qw0 + ql;
  const bool col_ok = hh < d.G && qi < T;
  const int qpos = pos0 + qi;                                // keys <= qpos
  bf16x8 qop[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col_ok)
      v = *reinterpret_cast<const uint4 *>(q + (((size_t)b * T + qi) * d.Hq + g * d.G + hh) * kHeadDim +
                                           8 * lg + 32 * s);
    qop[s] = as_bf16x8(v);
  }
  const float qscale = 0.08838834764831845f * 1.4426950408889634f;
  const float bscale = d.bias ? 1.4426950408889634f : 0.0f;
  const uint4 *kvg = reinterpret_cast<const uint4 *>(st.kv_dev + (size_t)p * d.NB_kv * kBlockElems);
  const float *tsp = st.tok_s + (size_t)p * d.tok_stride;
  const int koff0 = pa_tile_row(h, 0) * kPaKPitch + 16 * lg;
  const int koff1 = pa_tile_row(h, 1) * kPaKPitch + 16 * lg;

  // union cursor (uniform): the next set bit of orb at or after block `from`
  auto next_block = [&](int from) {
    for (int wi = from >> 5; wi < words; ++wi) {
      uint32_t u = orb[wi];
      if (wi == (from >> 5)) u &= ~0u << (from & 31);
      if (u) return 32 * wi + __builtin_ctz(u);
    }
    return -1;
  };
  // staging: thread t moves 16-byte pieces t + NT j of a block; pieces below
  // kBlock * 16 are K (row v / 16, dims 8 (v % 16)), the rest V
  static_assert(kVecs == 4 && NT * 2 == kBlock * kHeadDim / 8,
                "a thread stages two K pieces and two V pieces");
  uint4 pre0, pre1, pre2, pre3;                              // pieces t + NT j
  float spre = 0.0f;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  int blk = next_block(0);
  if (blk >= 0) {
    const uint4 *src = kvg + (size_t)blk * (kBlockElems * 2 / 16) + t;
    pre0 = src[0];
    pre1 = src[NT];
    pre2 = src[2 * NT];
    pre3 = src[3 * NT];
    if (t < kBlock) spre = tsp[blk * kBlock + t];
  }
  while (blk >= 0) {                                          // uniform
    __syncthreads();                                          // the last block is consumed
    {
      // pieces t and t + NT are K (row v / 16, dims 8 (v % 16)), t + 2 NT
      // and t + 3 NT the V part
      *reinterpret_cast<uint4 *>(kv_sh + (t >> 4) * kPaKPitch + 16 * (t & 15)) = pre0;
      *reinterpret_cast<uint4 *>(kv_sh + ((t + NT) >> 4) * kPaKPitch + 16 * (t & 15)) = pre1;
      *reinterpret_cast<uint4 *>(kv_sh + kPaKBytes + 16 * t) = pre2;
      *reinterpret_cast<uint4 *>(kv_sh + kPaKBytes + 16 * (t + NT)) = pre3;
      if (t < kBlock) s_sh[t] = spre;
    }
    __syncthreads();
    const int nxt = next_block(blk + 1);
    if (nxt >= 0) {
      const uint4 *src = kvg + (size_t)nxt * (kBlockElems * 2 / 16) + t;
      pre0 = src[0];
      pre1 = src[NT];
      pre2 = src[2 * NT];
      pre3 = src[3 * NT];
      if (t < kBlock) spre = tsp[nxt * kBlock + t];
    }
    const bool sel_col = col_ok && ((bits[ql * words + (blk >> 5)] >> (blk & 31)) & 1u);
    if (__ballot(sel_col) == 0) {                             // none of this wave's queries
      blk = nxt;
      continue;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 kk[2][4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kk[0][s] = *reinterpret_cast<const uint4 *>(kv_sh + half * 32 * kPaKPitch + koff0 + 64 * s);
        kk[1][s] = *reinterpret_cast<const uint4 *>(kv_sh + half * 32 * kPaKPitch + koff1 + 64 * s);
      }
      f32x4 acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[tt] = mfma16x16x32(as_bf16x8(kk[tt][s]), qop[s], acc[tt]);
      }
      const int key0 = blk * kBlock + 32 * half + 8 * lg;   // this lane's first key
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float sv = s_sh[32 * half + 8 * lg + m];
        const float lg2 = acc[m >> 2][m & 3] * qscale + sv * bscale;
        x[m] = (sel_col && key0 + m <= qpos) ? lg2 : -INFINITY;
        mx = fmaxf(mx, x[m]);
      }
      mx = xor32_max(xor16_max(mx));
      const float m_new = fmaxf(m_run, mx);
      const bool live = m_new != -INFINITY;                  // this column has a key so far
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      float psum = 0.0f;
      uint32_t phi[4], plo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 pm = live ? f32x2{__builtin_amdgcn_exp2f(x[2 * i] - m_new),
                                       __builtin_amdgcn_exp2f(x[2 * i + 1] - m_new)}
                              : f32x2{0.f, 0.f};
        psum += pm[0] + pm[1];
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(pm, bf16x2));
        const f32x2 back = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u)};
        phi[i] = hi;
        plo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pm - back, bf16x2));
      }
      if (live) m_run = m_new;
      l_run = l_run * alpha + psum;
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, uint4{phi[0], phi[1], phi[2], phi[3]});
      const bf16x8 blo = __builtin_bit_cast(bf16x8, uint4{plo[0], plo[1], plo[2], plo[3]});
      // once the columns' maxima settle (usually within the first blocks)
      // alpha is 1 in every lane and the rescale of O is skipped
      if (__ballot(alpha != 1.0f) != 0) {                    // uniform
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vt = as_bf16x8(*reinterpret_cast<const uint4 *>(
            kv_sh + kPaKBytes + half * 8192 + 16 * l + 1024 * dt));
        o[dt] = mfma16x16x32(vt, bhi, o[dt]);
        o[dt] = mfma16x16x32(vt, blo, o[dt]);
      }
    }
    blk = nxt;
  }
  if (__ballot(bad) && l == 0) atomicOr(st.status, NOSA_STATUS_BAD_SEL);

  // 3. normalise and write: lane (h, lg) holds O^T[16 dt + 4 lg + i][h]
  l_run = xor32_sum(xor16_sum(l_run));
  if (col_ok) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float *op = out + (((size_t)b * T + qi) * d.Hq + g * d.G + hh) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) op[16 * dt + 4 * lg + i] = o[dt][i] * inv;
  }
}

}  // namespace

hipError_t launch_prefill_select(const Dims &d, const nosa_state &st, const float *scores, int T,
                                 int pos0, int32_t *sel, int32_t *n_sel, hipStream_t s) {
  const int nb_out = blocks_for(pos0 + T);
  if (nb_out - d.n_sink <= 8 * 64)          // at most 8 candidates per lane of one wave
    prefill_select_kernel<64><<<dim3(T, d.P), 64, (size_t)d.NB_max, s>>>(
        d, st, scores, T, pos0, nb_out, sel, n_sel);
  else
    prefill_select_kernel<kTopkThreads><<<dim3(T, d.P), kTopkThreads, (size_t)d.NB_max, s>>>(
        d, st, scores, T, pos0, nb_out, sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_prefill_attend(const Dims &d, const nosa_state &st, const uint16_t *q, int T,
                                 int pos0, const int32_t *sel, const int32_t *n_sel, float *out,
                                 hipStream_t s) {
  const int QW = kPaWaves * pa_queries_per_wave(d.G);
  const size_t lds = (size_t)(QW + 1) * d.elig_words * sizeof(uint32_t);
  prefill_attend_kernel<<<dim3((T + QW - 1) / QW, d.P), kPaWaves * 64, lds, s>>>(
      d, st, q, T, pos0, sel, n_sel, out);
  return hipGetLastError();
}

}  // namespace nosa
