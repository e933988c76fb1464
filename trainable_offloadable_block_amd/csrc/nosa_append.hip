// Append + CompressK + eviction score (one decode step), and the bulk
// version used once to build the state from a prefilled context.
//
// Eviction head: s_j = softplus(v_j W1) W2, fp32 (aiwiki "NOSA", How NOSA
// works; l189 article, 2.1, eq. 4). CompressK: the mean of 32 keys with
// stride 16, summed exactly in fp64 and rounded once to bf16 (NOSA-1B
// 核心组件揭秘, 核心组件一). Block agnostic score: max over the chunks that
// overlap a block of the per-chunk mean score (l189 article, 2.1, eqs. 5-6).
#include "nosa_internal.h"

namespace nosa {
namespace {

// One KV head's W1 (32 KiB bf16) for a 128-thread group: 16 independent
// 16-byte loads per thread into registers, then into LDS (and a barrier).
constexpr int kW1Vecs = kHeadDim * kHeadDim * 2 / 16 / 128;
__device__ inline void load_w1(uint4 (&v)[kW1Vecs], const uint16_t *__restrict__ W1g) {
  const uint4 *src = reinterpret_cast<const uint4 *>(W1g);
#pragma unroll
  for (int j = 0; j < kW1Vecs; ++j) v[j] = src[threadIdx.x + 128 * j];
}
__device__ inline void store_w1(uint16_t *w1_sh, const uint4 (&v)[kW1Vecs]) {
  uint4 *dst = reinterpret_cast<uint4 *>(w1_sh);
#pragma unroll
  for (int j = 0; j < kW1Vecs; ++j) dst[threadIdx.x + 128 * j] = v[j];
  __syncthreads();
}
__device__ void stage_w1(uint16_t *w1_sh, const uint16_t *__restrict__ W1g) {
  uint4 v[kW1Vecs];
  load_w1(v, W1g);
  store_w1(w1_sh, v);
}

// s = softplus(v W1) W2 for one value vector held in LDS as fp32, with W1
// staged in LDS. Called by all 128 threads of a group; thread t owns hidden
// unit t. The summation order is fixed (e ascending, then a fixed reduction
// tree), so every caller gets the same bits for the same v.
__device__ float evict_score_128(const float *v_sh, const uint16_t *w1_sh,
                                 const uint16_t *__restrict__ W2g, float *red2) {
  const int t = threadIdx.x & 127;
  float acc = 0.0f;
#pragma unroll 16
  for (int e = 0; e < kHeadDim; ++e)
    acc = fmaf(v_sh[e], bf16_to_f32(w1_sh[e * kHeadDim + t]), acc);
  float x = softplus_f32(acc) * bf16_to_f32(W2g[t]);
  x = wave_sum(x);
  __syncthreads();                       // red2 may still be read by a caller
  if ((t & 63) == 0) red2[t >> 6] = x;
  __syncthreads();
  return red2[0] + red2[1];
}

// Zeroes one 32 KiB block with the workgroup's 128 threads; the barrier
// orders the zeros before the caller's token writes into the same block.
__device__ void clear_block(uint16_t *blk) {
  uint4 *b4 = reinterpret_cast<uint4 *>(blk);
  for (int i = threadIdx.x; i < kBlockElems * 2 / 16; i += blockDim.x) b4[i] = make_uint4(0, 0, 0, 0);
  __threadfence_block();
  __syncthreads();
}

// ------------------------------------------------------------- append
// grid (Hkv, B), block 128: one pair per workgroup, thread t = dim t.
__global__ __launch_bounds__(128) void append_kernel(
    Dims d, nosa_state st, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new) {
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int p = b * d.Hkv + g;
  __shared__ float v_sh[kHeadDim];
  __shared__ uint16_t k_sh[kHeadDim];
  __shared__ float red2[2];
  __shared__ int slot_sh;
  __shared__ __align__(16) uint16_t w1_sh[kHeadDim * kHeadDim];

  // loads that do not depend on the length first, so the kernel waits for
  // one memory round trip: the new key and value, this head's W1
  // (both go to LDS before the barrier, so neither load sinks into the
  // branch below, where they are used)
  const uint16_t kb_ld = k_new[p * kHeadDim + t];
  const uint16_t vb = v_new[p * kHeadDim + t];
  const int pos = st.seq_len[b];
  {
    uint4 w1v[kW1Vecs];
    load_w1(w1v, st.w1 + (size_t)g * kHeadDim * kHeadDim);
    v_sh[t] = bf16_to_f32(vb);
    k_sh[t] = kb_ld;
    store_w1(w1_sh, w1v);                // ends in a barrier
  }
  const uint16_t kb = k_sh[t];
  const bool ok = pos >= 0 && pos < d.max_context;
  if (ok) {
    const int L = pos + 1;
    const int blk = pos / kBlock, r = pos % kBlock;

    // 1. store K, V (K row-major, V in the block's tile order)
    if (!d.offload) {
      uint16_t *base = st.kv_dev + ((size_t)p * d.NB_max + blk) * kBlockElems;
      if (r == 0) clear_block(base);
      base[r * kHeadDim + t] = kb;
      base[kBlock * kHeadDim + v_index(r, t)] = vb;
    } else {
      uint16_t *hb = st.kv_host + ((size_t)p * d.NB_max + blk) * kBlockElems;
      hb[r * kHeadDim + t] = kb;
      hb[kBlock * kHeadDim + v_index(r, t)] = vb;
      int32_t *sob = st.slot_of_block + (size_t)p * d.NB_max;
      int32_t *bos = st.block_of_slot + (size_t)p * (d.k + 1);
      if (t == 0) slot_sh = sob[blk];
      __syncthreads();
      int slot = slot_sh;
      if (slot < 0 && r == 0) {          // this token opens a block: cache it
        __syncthreads();
        if (t == 0) slot_sh = 0x7fffffff;
        __syncthreads();
        for (int s = t; s <= d.k; s += blockDim.x)
          if (bos[s] < 0) atomicMin(&slot_sh, s);
        __syncthreads();
        slot = slot_sh == 0x7fffffff ? -1 : slot_sh;
        if (t == 0) {
          if (slot >= 0) {
            bos[slot] = blk;
            sob[blk] = slot;
          } else {
            atomicOr(st.status, NOSA_STATUS_BAD_SEL);
          }
        }
      }
      if (slot >= 0) {
        uint16_t *cb = st.kv_dev + ((size_t)p * (d.k + 1) + slot) * kBlockElems;
        if (r == 0) clear_block(cb);
        cb[r * kHeadDim + t] = kb;
        cb[kBlock * kHeadDim + v_index(r, t)] = vb;
      }
    }

    // 2. ring of the last 32 keys (feeds the chunk mean)
    uint16_t *ring = st.tail_keys + (size_t)p * kPoolKernel * kHeadDim;
    ring[(pos % kPoolKernel) * kHeadDim + t] = kb;

    // 3. eviction score of the new token
    const float s = evict_score_128(v_sh, w1_sh, st.w2 + (size_t)g * kHeadDim, red2);
    float *tok_s = st.tok_s + (size_t)p * d.tok_stride;
    if (t == 0) tok_s[pos] = s;

    // 4. a chunk completes when L >= 32 and (L - 32) % 16 == 0
    if (L >= kPoolKernel && (L - kPoolKernel) % kPoolStride == 0) {
      const int i = (L - kPoolKernel) / kPoolStride;
      double sum = 0.0;                  // exact for bf16 inputs of sane range
      for (int j = 0; j < kPoolKernel; ++j) {
        const int tok = pos - (kPoolKernel - 1) + j;
        const uint16_t kv = tok == pos ? kb : ring[(tok % kPoolKernel) * kHeadDim + t];
        sum += (double)bf16_to_f32(kv);
      }
      st.ckey[((size_t)p * d.C_max + i) * kHeadDim + t] =
          f64_to_bf16_rne(sum * (1.0 / kPoolKernel));
      if (t < 64) {                      // wave 0: mean eviction score
        double se = 0.0;
        if (t < kPoolKernel) {
          const int tok = pos - (kPoolKernel - 1) + t;
          se = tok == pos ? (double)s : (double)tok_s[tok];
        }
        se = wave_sum(se);
        if (t == 0) {
          const float em = (float)(se * (1.0 / kPoolKernel));
          float *ce = st.chunk_e + (size_t)p * d.C_max;
          ce[i] = em;
          if (i % 4 == 3) {              // block (i-3)/4 now has all chunks
            const int bb = (i - 3) / 4;
            float m = em;
            for (int c = (bb > 0 ? 4 * bb - 1 : 0); c < i; ++c) m = fmaxf(m, ce[c]);
            st.blk_e[(size_t)p * d.NB_max + bb] = m;
          }
        }
      }
    }
  }
  // last workgroup of this sequence advances its length. Every workgroup
  // has consumed seq_len[b] (all its addresses depend on it) before it
  // arrives, so no fence is needed (a device-scope fence would write back
  // the XCD's whole L2).
  __syncthreads();
  if (t == 0) {
    if (!ok) atomicOr(st.status, NOSA_STATUS_CAPACITY);
    const int old = atomicAdd(&st.arrive[b], 1);
    if (old == d.Hkv - 1) {
      st.arrive[b] = 0;
      if (ok) st.seq_len[b] = pos + 1;
    }
  }
}

// ------------------------------------------------------------- prefill
// Eviction scores of every prefilled token. grid (blocks, P), block 128:
// the V half of one 64-token block is staged in LDS, then one token at a
// time goes through the same eviction head as append.
__global__ __launch_bounds__(128) void prefill_scores_kernel(Dims d, nosa_state st) {
  const int blk = blockIdx.x, p = blockIdx.y, t = threadIdx.x;
  const int b = p / d.Hkv, g = p % d.Hkv;
  const int L = min(st.seq_len[b], d.max_context);
  if (blk * kBlock >= L) return;
  __shared__ uint4 vt_sh[kBlock * kHeadDim * 2 / 16];   // V part, 16 KiB
  __shared__ float v_sh[kHeadDim];
  __shared__ float red2[2];
  __shared__ __align__(16) uint16_t w1_sh[kHeadDim * kHeadDim];
  const uint16_t *src = (d.offload ? st.kv_host : st.kv_dev) +
                        ((size_t)p * d.NB_max + blk) * kBlockElems + kBlock * kHeadDim;
  const uint4 *src4 = reinterpret_cast<const uint4 *>(src);
  for (int i = t; i < kBlock * kHeadDim * 2 / 16; i += blockDim.x) vt_sh[i] = src4[i];
  stage_w1(w1_sh, st.w1 + (size_t)g * kHeadDim * kHeadDim);   // ends in a barrier
  const uint16_t *vt = reinterpret_cast<const uint16_t *>(vt_sh);
  const int n = min(kBlock, L - blk * kBlock);
  float *tok_s = st.tok_s + (size_t)p * d.tok_stride;
  for (int r = 0; r < n; ++r) {
    v_sh[t] = bf16_to_f32(vt[v_index(r, t)]);
    __syncthreads();
    const float s = evict_score_128(v_sh, w1_sh, st.w2 + (size_t)g * kHeadDim, red2);
    if (t == 0) tok_s[blk * kBlock + r] = s;
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
    double sum = 0.0;
    for (int j = 0; j < kPoolKernel; ++j) {
      const int tok = i * kPoolStride + j;
      const uint16_t *row = kvb + ((size_t)p * d.NB_max + tok / kBlock) * kBlockElems +
                            (tok % kBlock) * kHeadDim;
      sum += (double)bf16_to_f32(row[t]);
    }
    st.ckey[((size_t)p * d.C_max + i) * kHeadDim + t] =
        f64_to_bf16_rne(sum * (1.0 / kPoolKernel));
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
                     ((size_t)p * d.NB_max + L / kBlock) * kBlockElems;
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
      const uint16_t *row = kvb + ((size_t)p * d.NB_max + tok / kBlock) * kBlockElems +
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
    prefill_scores_kernel<<<dim3(nbl, d.P), 128, 0, s>>>(d, st);
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
