// Device parts of the append step, shared by the append kernel and the fused
// append + select kernel.
//
// Eviction head: s_j = softplus(v_j W1) W2, fp32 (aiwiki "NOSA", How NOSA
// works; l189 article, 2.1, eq. 4). CompressK: the mean of 32 keys with
// stride 16, summed exactly in fp64 and rounded once to bf16 (NOSA-1B
// 核心组件揭秘, 核心组件一). Block agnostic score: max over the chunks that
// overlap a block of the per-chunk mean score (l189 article, 2.1, eqs. 5-6).
#pragma once

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
// staged in LDS. Called by all threads of a group of 128 or more; thread
// t < 128 owns hidden unit t. The summation order is fixed (e ascending, then a fixed reduction
// tree), so every caller gets the same bits for the same v.
__device__ __forceinline__ float evict_score_128(const float *v_sh, const uint16_t *w1_sh,
                                 const uint16_t *__restrict__ W2g, float *red2) {
  const int t = threadIdx.x & 127;
  float acc = 0.0f;
#pragma unroll 16
  for (int e = 0; e < kHeadDim; ++e)
    acc = fmaf(v_sh[e], bf16_to_f32(w1_sh[e * kHeadDim + t]), acc);
  float x = softplus_f32(acc) * bf16_to_f32(W2g[t]);
  x = wave_sum(x);
  __syncthreads();                       // red2 may still be read by a caller
  if (threadIdx.x < kHeadDim && (t & 63) == 0) red2[t >> 6] = x;
  __syncthreads();
  return red2[0] + red2[1];
}

// Zeroes one 32 KiB block with the workgroup's 128 threads; the barrier
// orders the zeros before the caller's token writes into the same block.
__device__ __forceinline__ void clear_block(uint16_t *blk) {
  uint4 *b4 = reinterpret_cast<uint4 *>(blk);
  for (int i = threadIdx.x; i < kBlockElems * 2 / 16; i += blockDim.x) b4[i] = make_uint4(0, 0, 0, 0);
  __threadfence_block();
  __syncthreads();
}

// LDS of one pair's append step.
struct AppendLds {
  float v_sh[kHeadDim];
  uint16_t k_sh[kHeadDim];
  float red2[2];
  int slot_sh;
  __align__(16) uint16_t w1_sh[kHeadDim * kHeadDim];
};

// Appends the token at position pos of pair p = b * Hkv + g with a group of
// NT >= 128 threads (thread t < 128 owns dim t): K and V into the pool
// (resident) or into the host store and the pair's cache slot (offload; a
// token that opens a block takes a free slot), the tail ring, the token's
// eviction score and, when the token completes a chunk, the chunk's
// compressed key, its mean score and, when that
// completes a block, the block's agnostic score (the key and the block score
// stored device-coherently when `coherent`, for readers in the same launch). Does nothing when pos is
// outside [0, max_context). Returns the completed chunk's index, or -1.
// Loads that do not depend on pos are issued first. Called by all NT
// threads.
template <int NT>
__device__ __forceinline__ int append_pair(const Dims &d, const nosa_state &st, const uint16_t *__restrict__ k_new,
                           const uint16_t *__restrict__ v_new, int b, int g, int pos,
                           bool coherent, AppendLds &sh) {
  const int t = threadIdx.x, p = b * d.Hkv + g;
  const bool dim = t < kHeadDim;
  // the new key and value and this head's W1 first (the key and value go to
  // LDS before the barrier, so neither load sinks into the branch below)
  uint16_t kb_ld = 0, vb = 0;
  if (dim) {
    kb_ld = k_new[p * kHeadDim + t];
    vb = v_new[p * kHeadDim + t];
  }
  {
    constexpr int NV = kHeadDim * kHeadDim * 2 / 16 / NT;
    const uint4 *src = reinterpret_cast<const uint4 *>(st.w1 + (size_t)g * kHeadDim * kHeadDim);
    uint4 w1v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) w1v[j] = src[t + NT * j];
    if (dim) {
      sh.v_sh[t] = bf16_to_f32(vb);
      sh.k_sh[t] = kb_ld;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(sh.w1_sh);
#pragma unroll
    for (int j = 0; j < NV; ++j) dst[t + NT * j] = w1v[j];
    __syncthreads();
  }
  const uint16_t kb = dim ? sh.k_sh[t] : 0;
  if (pos < 0 || pos >= d.max_context) return -1;          // uniform
  const int L = pos + 1;
  const int blk = pos / kBlock, r = pos % kBlock;

  // 1. store K, V (K row-major, V in the block's tile order)
  if (!d.offload) {
    uint16_t *base = st.kv_dev + ((size_t)p * d.NB_kv + blk) * kBlockElems;
    if (r == 0) clear_block(base);
    if (dim) {
      base[r * kHeadDim + t] = kb;
      base[kBlock * kHeadDim + v_index(r, t)] = vb;
    }
  } else {
    // offload: the token goes to its block's cache slot; the host store gets
    // the whole block, in coalesced 16-byte writes, when its last token
    // arrives (a block stays cached until then: the window holds it). A token
    // whose block is not cached (before the first fetch) goes to the host
    // store directly.
    uint16_t *hb = st.kv_host + ((size_t)p * d.NB_kv + blk) * kBlockElems;
    int32_t *sob = st.slot_of_block + (size_t)p * d.NB_max;
    int32_t *bos = st.block_of_slot + (size_t)p * (d.k + 1);
    if (t == 0) sh.slot_sh = sob[blk];
    __syncthreads();
    int slot = sh.slot_sh;
    if (slot < 0 && r == 0) {            // this token opens a block: cache it
      __syncthreads();
      if (t == 0) sh.slot_sh = 0x7fffffff;
      __syncthreads();
      for (int s = t; s <= d.k; s += NT)
        if (bos[s] < 0) atomicMin(&sh.slot_sh, s);
      __syncthreads();
      slot = sh.slot_sh == 0x7fffffff ? -1 : sh.slot_sh;
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
      if (dim) {
        cb[r * kHeadDim + t] = kb;
        cb[kBlock * kHeadDim + v_index(r, t)] = vb;
      }
      if (r == kBlock - 1) {               // complete: write it back
        __syncthreads();
        const uint4 *c4 = reinterpret_cast<const uint4 *>(cb);
        uint4 *h4 = reinterpret_cast<uint4 *>(hb);
        for (int i = t; i < kBlockElems * 2 / 16; i += NT) h4[i] = c4[i];
      }
    } else if (dim) {
      hb[r * kHeadDim + t] = kb;
      hb[kBlock * kHeadDim + v_index(r, t)] = vb;
    }
  }

  // 2. ring of the last 32 keys (feeds the chunk mean)
  uint16_t *ring = st.tail_keys + (size_t)p * kPoolKernel * kHeadDim;
  if (dim) ring[(pos % kPoolKernel) * kHeadDim + t] = kb;

  // 3. eviction score of the new token
  const float s = evict_score_128(sh.v_sh, sh.w1_sh, st.w2 + (size_t)g * kHeadDim, sh.red2);
  float *tok_s = st.tok_s + (size_t)p * d.tok_stride;
  if (t == 0) tok_s[pos] = s;

  // 4. a chunk completes when L >= 32 and (L - 32) % 16 == 0
  if (L < kPoolKernel || (L - kPoolKernel) % kPoolStride != 0) return -1;
  const int i = (L - kPoolKernel) / kPoolStride;
  if (dim) {
    const uint16_t c = mean32_bf16([&](int j) -> uint16_t {
      const int tok = pos - (kPoolKernel - 1) + j;
      return tok == pos ? kb : ring[(tok % kPoolKernel) * kHeadDim + t];
    });
    uint16_t *row = st.ckey + ((size_t)p * d.C_max + i) * kHeadDim;
    if (coherent) {
      const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
          row, (short)0, kHeadDim * 2, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b16(c, rr, 2 * t, 0, 16);   // sc1: device-coherent
    } else {
      row[t] = c;
    }
  }
  if (t < 64) {                          // wave 0: mean eviction score
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
      if (i % 4 == 3) {                  // block (i-3)/4 now has all chunks
        const int bb = (i - 3) / 4;
        float m = em;
        for (int c = (bb > 0 ? 4 * bb - 1 : 0); c < i; ++c) m = fmaxf(m, ce[c]);
        float *dst = st.blk_e + (size_t)p * d.NB_max + bb;
        if (coherent)
          __hip_atomic_store(dst, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = m;
      }
    }
  }
  return i;
}

}  // namespace
}  // namespace nosa
