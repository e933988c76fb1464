// Sparse prefill in NOSA_S's style (aiwiki "NOSA", Results: sparse in both
// phases): every prompt query selects and attends as a decode step at its own
// length would, with every candidate block eligible (the never-reselect state
// begins with decoding; aiwiki "NOSA", How NOSA works).
//
// prefill_select_kernel: grid (queries, pairs), one workgroup per query:
//   stage 1 takes the k_q candidates of highest block score (from
//   nosa_prefill_block_scores), stage 2 the k_e' others of highest agnostic
//   score; the ascending list of sink, window and selected blocks.
// prefill_attend_kernel: grid (query groups, pairs), 4 waves; a wave takes
//   16 / Gp consecutive queries (16 MFMA columns of (query, head)), forms the
//   union of their selections in LDS and streams those blocks half by half:
//   logits S^T = K Q^T on MFMA, a column is masked where its query did not
//   select the block or the key lies past the query's position, an online
//   softmax per column in the log2 domain with the eviction-score bias, and
//   O^T += V^T P^T on MFMA (P split into bf16 hi + lo). Resident KV only.
#include "nosa_select_dev.h"

namespace nosa {
namespace {

__host__ __device__ inline int pa_rows(int G) { return G <= 4 ? 4 : (G <= 8 ? 8 : 16); }
constexpr int kPaWaves = 4;

// ---------------------------------------------------------------- select
template <int R>
__device__ __forceinline__ void pf_stages(const Dims &d, const float *__restrict__ sc,
                                          const float *__restrict__ be, int n_cand,
                                          uint8_t *kind, TopkLds &tk) {
  const int t = threadIdx.x;
  if (d.k_q > 0) {
    uint64_t kq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + kTopkThreads * r, bb = d.n_sink + i;
      kq[r] = i < n_cand ? compose_key(sc[bb], bb) : 0;
    }
    wg_topk(kq, d.k_q, d.n_sink, kind, NOSA_KIND_QUERY, tk);
    __syncthreads();
  }
  if (d.k_e_dyn > 0) {
    uint64_t ke[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = t + kTopkThreads * r, bb = d.n_sink + i;
      ke[r] = (i < n_cand && kind[bb] != NOSA_KIND_QUERY) ? compose_key(be[bb], bb) : 0;
    }
    wg_topk(ke, d.k_e_dyn, d.n_sink, kind, NOSA_KIND_AGNOSTIC, tk);
  }
}

__global__ __launch_bounds__(kTopkThreads) void prefill_select_kernel(
    Dims d, nosa_state st, const float *__restrict__ scores, int T, int pos0, int nb_out,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel) {
  extern __shared__ __align__(16) uint8_t kind[];          // [NB_max]
  __shared__ TopkLds tk;
  __shared__ int cnt_sh[2][kTopkThreads / 64];
  const int qi = blockIdx.x, p = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int L = pos0 + qi + 1;
  const int nb = blocks_for(L);
  const int win_lo = max(d.n_sink, nb - d.n_win);
  const int n_cand = max(0, win_lo - d.n_sink);
  for (int bb = t; bb < nb; bb += kTopkThreads)
    kind[bb] = bb < d.n_sink ? NOSA_KIND_SINK : (bb >= win_lo ? NOSA_KIND_WINDOW : NOSA_KIND_NONE);
#pragma unroll
  for (int i = 0; i < kTopkBins / kTopkThreads; ++i) {
    tk.hist[0][t + kTopkThreads * i] = 0;
    tk.hist[1][t + kTopkThreads * i] = 0;
  }
  __syncthreads();
  if (n_cand > 0) {                                         // uniform
    const float *sc = scores + ((size_t)p * T + qi) * nb_out;
    const float *be = st.blk_e + (size_t)p * d.NB_max;
    const int m = (n_cand + kTopkThreads - 1) / kTopkThreads;
    if (m <= 1) pf_stages<1>(d, sc, be, n_cand, kind, tk);
    else if (m <= 2) pf_stages<2>(d, sc, be, n_cand, kind, tk);
    else if (m <= 4) pf_stages<4>(d, sc, be, n_cand, kind, tk);
    else if (m <= 8) pf_stages<8>(d, sc, be, n_cand, kind, tk);
    else pf_stages<kMaxCandPerThread>(d, sc, be, n_cand, kind, tk);
  }
  __syncthreads();
  // ascending list: ballot + prefix count per 256 blocks
  int32_t *sp = sel + ((size_t)p * T + qi) * d.k;
  int running = 0;
  for (int base = 0; base < nb; base += kTopkThreads) {      // uniform
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
    if (in && off < d.k) sp[off] = bb;
    running += tot;
  }
  for (int j = running + t; j < d.k; j += kTopkThreads) sp[j] = -1;
  if (t == 0) n_sel[(size_t)p * T + qi] = min(running, d.k);
}

// ---------------------------------------------------------------- attend
constexpr int kPaMaxQ = 4;                 // queries per wave (Gp = 4)
constexpr int kPaMaxWords = kMaxContext / kBlock / 32;   // bitmap words
constexpr int kPaMaxUnion = kPaMaxQ * kMaxK;

// A-row r of tile t <-> key 8*(r/4) + 4*t + (r%4) of a 32-key half, so that
// lane group j holds keys 8j .. 8j+7 of the half (the decode kernel's order).
__device__ inline int pa_tile_row(int r, int t) { return 8 * (r >> 2) + 4 * t + (r & 3); }

__global__ __launch_bounds__(kPaWaves * 64) void prefill_attend_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ q, int T, int pos0,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ n_sel,
    float *__restrict__ out) {
  __shared__ uint32_t bits[kPaWaves][kPaMaxQ][kPaMaxWords];
  __shared__ int ulist[kPaWaves][kPaMaxUnion];
  __shared__ uint8_t umask[kPaWaves][kPaMaxUnion];
  const int p = blockIdx.y, b = p / d.Hkv, g = p % d.Hkv;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l & 15, lg = l >> 4;
  const int Gp = pa_rows(d.G), QT = 16 / Gp;
  const int q0 = (blockIdx.x * kPaWaves + w) * QT;
  const int words = d.elig_words;

  // 1. the wave's queries' selections as bitmaps, then their union
  for (int qq = 0; qq < QT; ++qq)
    for (int i = l; i < words; i += 64) bits[w][qq][i] = 0u;
  __syncthreads();
  bool bad = false;
  for (int qq = 0; qq < QT; ++qq) {
    const int qi = q0 + qq;
    if (qi >= T) break;
    const int ns = max(0, min(n_sel[(size_t)p * T + qi], d.k));
    for (int e = l; e < ns; e += 64) {
      const int blk = sel[((size_t)p * T + qi) * d.k + e];
      if (blk >= 0 && blk < d.NB_max && blk * kBlock <= pos0 + qi)
        atomicOr(&bits[w][qq][blk >> 5], 1u << (blk & 31));
      else
        bad = true;
    }
  }
  __syncthreads();
  int n_union = 0;
  for (int base = 0; base < words; base += 64) {             // wave-uniform
    const int wi = base + l;
    uint32_t u = 0u;
    if (wi < words)
      for (int qq = 0; qq < QT; ++qq) u |= bits[w][qq][wi];
    const uint32_t cnt = __popc(u);
    const uint32_t incl = wave_incl_scan(cnt);
    int off = n_union + static_cast<int>(incl - cnt);
    while (u) {
      const int bit = __builtin_ctz(u);
      u &= u - 1u;
      const int blk = 32 * wi + bit;
      uint8_t m = 0;
      for (int qq = 0; qq < QT; ++qq) m |= ((bits[w][qq][wi] >> bit) & 1u) << qq;
      if (off < kPaMaxUnion) {
        ulist[w][off] = blk;
        umask[w][off] = m;
      }
      ++off;
    }
    n_union += static_cast<int>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  }
  n_union = min(n_union, kPaMaxUnion);
  __syncthreads();

  // 2. this lane's column: query qq = h / Gp, head hh = h % Gp
  const int qq = h / Gp, hh = h % Gp, qi = q0 + qq;
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
  const char *kvp = reinterpret_cast<const char *>(st.kv_dev + (size_t)p * d.NB_max * kBlockElems);
  const float *tsp = st.tok_s + (size_t)p * d.tok_stride;
  const int koff0 = pa_tile_row(h, 0) * kHeadDim * 2 + 16 * lg;
  const int koff1 = pa_tile_row(h, 1) * kHeadDim * 2 + 16 * lg;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < 2 * n_union; ++j) {                    // wave-uniform
    const int blk = ulist[w][j >> 1], half = j & 1;
    const bool sel_col = col_ok && ((umask[w][j >> 1] >> qq) & 1);
    const char *kb = kvp + (size_t)blk * (kBlockElems * 2) + half * (32 * kHeadDim * 2);
    const char *vb = kvp + (size_t)blk * (kBlockElems * 2) + kBlock * kHeadDim * 2 + half * 8192;
    uint4 kk[2][4], vv[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kk[0][s] = *reinterpret_cast<const uint4 *>(kb + koff0 + 64 * s);
      kk[1][s] = *reinterpret_cast<const uint4 *>(kb + koff1 + 64 * s);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vv[dt] = *reinterpret_cast<const uint4 *>(vb + 16 * l + 1024 * dt);
    const int key_base = blk * kBlock + 32 * half;
    const float sv_lane = tsp[key_base + (l & 31)];
    f32x4 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[t] = mfma16x16x32(as_bf16x8(kk[t][s]), qop[s], acc[t]);
    }
    const int key0 = key_base + 8 * lg;                      // this lane's first key
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float sv = __shfl(sv_lane, 8 * lg + m, 64);
      const float lg2 = acc[m >> 2][m & 3] * qscale + sv * bscale;
      x[m] = (sel_col && key0 + m <= qpos) ? lg2 : -INFINITY;
      mx = fmaxf(mx, x[m]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const bool live = m_new != -INFINITY;                    // this column has a key so far
    const float alpha = live ? exp2f(m_run - m_new) : 1.0f;
    float psum = 0.0f;
    uint32_t phi[4], plo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 pm = live ? f32x2{exp2f(x[2 * i] - m_new), exp2f(x[2 * i + 1] - m_new)}
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
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      o[dt] *= alpha;
      o[dt] = mfma16x16x32(as_bf16x8(vv[dt]), bhi, o[dt]);
      o[dt] = mfma16x16x32(as_bf16x8(vv[dt]), blo, o[dt]);
    }
  }
  if (__ballot(bad) && l == 0) atomicOr(st.status, NOSA_STATUS_BAD_SEL);

  // 3. normalise and write: lane (h, lg) holds O^T[16 dt + 4 lg + i][h]
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
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
  prefill_select_kernel<<<dim3(T, d.P), kTopkThreads, (size_t)d.NB_max, s>>>(
      d, st, scores, T, pos0, blocks_for(pos0 + T), sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_prefill_attend(const Dims &d, const nosa_state &st, const uint16_t *q, int T,
                                 int pos0, const int32_t *sel, const int32_t *n_sel, float *out,
                                 hipStream_t s) {
  const int QG = kPaWaves * (16 / pa_rows(d.G));
  prefill_attend_kernel<<<dim3((T + QG - 1) / QG, d.P), kPaWaves * 64, 0, s>>>(
      d, st, q, T, pos0, sel, n_sel, out);
  return hipGetLastError();
}

}  // namespace nosa
