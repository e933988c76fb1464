// Append + CompressK + eviction score (one decode step), and the bulk
// version used once to build the state from a prefilled context (the
// eviction head of every prefilled token as a dense MFMA product).
//
// Eviction head: s_j = softplus(v_j W1) W2, fp32 (aiwiki "NOSA", How NOSA
// works; l189 article, 2.1, eq. 4). CompressK: the mean of 32 keys with
// stride 16, summed exactly in fp64 and rounded once to bf16 (NOSA-1B
// 核心组件揭秘, 核心组件一). Block agnostic score: max over the chunks that
// overlap a block of the per-chunk mean score (l189 article, 2.1, eqs. 5-6).
#include "nosa_append_dev.h"

namespace nosa {
namespace {

// ------------------------------------------------------------- append
// grid (Hkv, B), block 128: one pair per workgroup, thread t = dim t.
__global__ __launch_bounds__(128) void append_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new) {
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  __shared__ AppendLds sh;
  const int pos = st.seq_len[b];
  append_pair<128>(d, st, k_new, v_new, b, g, pos, false, sh);
  // last workgroup of this sequence advances its length. Every workgroup
  // has consumed seq_len[b] (all its addresses depend on it) before it
  // arrives, so no fence is needed (a device-scope fence would write back
  // the XCD's whole L2).
  __syncthreads();
  if (t == 0) {
    const bool ok = pos >= 0 && pos < d.max_context;
    if (!ok) atomicOr(st.status, NOSA_STATUS_CAPACITY);
    const int old = atomicAdd(&st.arrive[b], 1);
    if (old == d.Hkv - 1) {
      st.arrive[b] = 0;
      if (ok) st.seq_len[b] = pos + 1;
    }
  }
}

// ------------------------------------------------------------- prefill
// Eviction scores of every prefilled token as one dense product on MFMA:
// S = V W1 (tokens x hidden, bf16 in, fp32 accumulate), then
// s = softplus(S) W2 per token. grid (ceil(blocks / kPfBlocks), P), 4 waves:
// W1 is staged once per workgroup, transposed to [hidden][input] so a lane's
// 8 consecutive inputs are one 16-byte LDS read; each 64-token block's V part
// (tile order) is staged as [token][dim]; wave w takes tokens 16w .. 16w+15
// of the block against all 128 hidden units (8 column tiles x 4 k-steps).
constexpr int kPfBlocks = 8;                 // 64-token blocks per workgroup
constexpr int kPfPad = kHeadDim + 8;         // LDS row pitch (elements)

__global__ __launch_bounds__(256) void prefill_scores_kernel(Dims d, nosa_state st) {
  const int p = blockIdx.y, t = threadIdx.x;
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int L = min(st.seq_len[b], d.max_context);
  const int blk0 = blockIdx.x * kPfBlocks;
  if (blk0 * kBlock >= L) return;
  __shared__ __align__(16) uint16_t w1t[kHeadDim * kPfPad];   // [hidden][input]
  __shared__ __align__(16) uint16_t vs[kBlock * kPfPad];      // [token][dim]
  __shared__ float w2s[kHeadDim];
  const int w = t >> 6, l = t & 63, lr = l & 15, lg = l >> 4;

  {   // W1 [input][hidden] -> w1t[hidden][input]
    const uint4 *src = reinterpret_cast<const uint4 *>(st.w1 + (size_t)g * kHeadDim * kHeadDim);
#pragma unroll
    for (int j = 0; j < kHeadDim * kHeadDim / 8 / 256; ++j) {
      const int i = t + 256 * j;             // 16-byte piece: input e, hidden 8h8 .. 8h8+7
      const int e = i >> 4, h8 = i & 15;
      const uint4 v = src[i];
      const uint16_t *x = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
      for (int q = 0; q < 8; ++q) w1t[(8 * h8 + q) * kPfPad + e] = x[q];
    }
    if (t < kHeadDim) w2s[t] = bf16_to_f32(st.w2[(size_t)g * kHeadDim + t]);
  }
  const uint16_t *kvb = d.offload ? st.kv_host : st.kv_dev;
  float *tok_s = st.tok_s + (size_t)p * d.tok_stride;
  const int blk_end = min(blk0 + kPfBlocks, blocks_for(L));
  for (int blk = blk0; blk < blk_end; ++blk) {
    __syncthreads();                         // W1 staged / previous block's vs consumed
    {   // V part, tile order -> vs[token][dim]
      const uint4 *src = reinterpret_cast<const uint4 *>(
          kvb + ((size_t)p * d.NB_kv + blk) * kBlockElems + kBlock * kHeadDim);
#pragma unroll
      for (int j = 0; j < kBlock * kHeadDim / 8 / 256; ++j) {
        const int gi = t + 256 * j;           // 8 tokens of one dim
        const int half = gi >> 9, ct = (gi >> 6) & 7, tg = (gi >> 4) & 3, c16 = gi & 15;
        const int tok0 = 32 * half + 8 * tg, dim = 16 * ct + c16;
        const uint4 v = src[gi];
        const uint16_t *x = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
        for (int q = 0; q < 8; ++q) vs[(tok0 + q) * kPfPad + dim] = x[q];
      }
    }
    __syncthreads();
    bf16x8 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(&vs[(16 * w + lr) * kPfPad + 32 * ks + 8 * lg]));
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 bop = as_bf16x8(
            *reinterpret_cast<const uint4 *>(&w1t[(16 * ct + lr) * kPfPad + 32 * ks + 8 * lg]));
        acc = mfma16x16x32(a[ks], bop, acc);
      }
      // lane (lr, lg): tokens 16w + 4lg + i against hidden unit 16ct + lr
      const float w2v = w2s[16 * ct + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = fmaf(softplus_f32(acc[i]), w2v, part[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = part[i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
      const int tok = blk * kBlock + 16 * w + 4 * lg + i;
      if (lr == 0 && tok < L) tok_s[tok] = x;
    }
  }
}

// Compressed keys and chunk means of every complete chunk. grid (blocks, P),
// block 128: workgroup blk handles chunks 4*blk .. 4*blk+3.
__global__ __launch_bounds__(128) void prefill_chunks_kernel(Dims d, nosa_state st) {
  const int blk = blockIdx.x, p = blockIdx.y, t = threadIdx.x;
  const int b = p / d.Hkv;
  const int L = min(st.seq_len[b], d.max_context);
  const int C = chunks_for(L);
  const uint16_t *kvb = d.offload ? st.kv_host : st.kv_dev;
  const float *tok_s = st.tok_s + (size_t)p * d.tok_stride;
  for (int c = 0; c < 4; ++c) {
    const int i = 4 * blk + c;
    if (i >= C) return;
    st.ckey[((size_t)p * d.C_max + i) * kHeadDim + t] = mean32_bf16([&](int j) -> uint16_t {
      const int tok = i * kPoolStride + j;
      return kvb[((size_t)p * d.NB_kv + tok / kBlock) * kBlockElems +
                 (tok % kBlock) * kHeadDim + t];
    });
    if (t < 64) {
      double se = t < kPoolKernel ? (double)tok_s[i * kPoolStride + t] : 0.0;
      se = wave_sum(se);
      if (t == 0) st.chunk_e[(size_t)p * d.C_max + i] = (float)(se * (1.0 / kPoolKernel));
    }
  }
}

// Block scores, eligibility, tail ring, cache maps, counters.
// grid (ceil(max(NB_max, words)/128), P), block 128.
__global__ __launch_bounds__(128) void prefill_finish_kernel(Dims d, nosa_state st) {
  const int p = blockIdx.y, t = threadIdx.x;
  const int b = p / d.Hkv;
  const int L = max(0, min(st.seq_len[b], d.max_context));
  const int C = chunks_for(L);
  const int idx = blockIdx.x * blockDim.x + t;
  // E_b for every block whose chunks 4b-1 .. 4b+3 are all complete
  if (idx < d.NB_max && 4 * idx + 3 < C) {
    const float *ce = st.chunk_e + (size_t)p * d.C_max;
    float m = ce[4 * idx + 3];
    for (int c = (idx > 0 ? 4 * idx - 1 : 0); c < 4 * idx + 3; ++c) m = fmaxf(m, ce[c]);
    st.blk_e[(size_t)p * d.NB_max + idx] = m;
  }
  if (idx < d.elig_words) st.eligible[(size_t)p * d.elig_words + idx] = 0xFFFFFFFFu;
  if (d.offload) {
    if (idx < d.NB_max) st.slot_of_block[(size_t)p * d.NB_max + idx] = -1;
    if (idx <= d.k) st.block_of_slot[(size_t)p * (d.k + 1) + idx] = -1;
  }
  if (L % kBlock) {
    // tail of the last, partial block: K and V of the positions past L read 0
    uint16_t *base = (d.offload ? st.kv_host : st.kv_dev) +
                     ((size_t)p * d.NB_kv + L / kBlock) * kBlockElems;
    const int r0 = L % kBlock, n = (kBlock - r0) * kHeadDim;
    for (int i = idx; i < n; i += gridDim.x * blockDim.x) {
      const int tok = r0 + i / kHeadDim, dim = i % kHeadDim;
      base[tok * kHeadDim + dim] = 0;                                // K
      base[kBlock * kHeadDim + v_index(tok, dim)] = 0;               // V
    }
  }
  if (blockIdx.x == 0) {
    // ring slot j holds the key of the latest position congruent to j mod 32
    const uint16_t *kvb = d.offload ? st.kv_host : st.kv_dev;
    uint16_t *ring = st.tail_keys + (size_t)p * kPoolKernel * kHeadDim;
    for (int j = 0; j < kPoolKernel; ++j) {
      const int tok = L - kPoolKernel + j;
      if (tok < 0) continue;
      const uint16_t *row = kvb + ((size_t)p * d.NB_kv + tok / kBlock) * kBlockElems +
                            (tok % kBlock) * kHeadDim;
      ring[(tok % kPoolKernel) * kHeadDim + t] = row[t];
    }
    if (p == 0) {
      for (int i = t; i < d.B; i += blockDim.x) st.arrive[i] = 0;
      if (t == 0) st.status[0] = 0u;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const Dims &d, const nosa_state &st, int max_len,
                          hipStream_t s) {
  const int nbl = blocks_for(max_len);
  if (nbl > 0) {
    prefill_scores_kernel<<<dim3((nbl + kPfBlocks - 1) / kPfBlocks, d.P), 256, 0, s>>>(d, st);
    prefill_chunks_kernel<<<dim3(nbl, d.P), 128, 0, s>>>(d, st);
  }
  const int span = d.NB_max > d.elig_words ? d.NB_max : d.elig_words;
  const int span2 = span > d.k + 1 ? span : d.k + 1;
  prefill_finish_kernel<<<dim3((span2 + 127) / 128, d.P), 128, 0, s>>>(d, st);
  return hipGetLastError();
}

hipError_t launch_append(const Dims &d, const nosa_state &st,
                         const uint16_t *k_new, const uint16_t *v_new,
                         hipStream_t s) {
  append_kernel<<<dim3(d.Hkv, d.B), 128, 0, s>>>(d, st, k_new, v_new);
  return hipGetLastError();
}

}  // namespace nosa
