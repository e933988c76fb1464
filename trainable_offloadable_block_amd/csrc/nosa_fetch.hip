// Delta fetch for offloaded KV (aiwiki "NOSA", NOSI: the inference system:
// a set-difference kernel between the previous and current selection so only
// changed blocks move, and a kernel that reads pinned host memory directly;
// SparDA article on aliyun, KV 预取的运行时实现: the GPU keeps the previous
// step's top-k blocks per layer and fetches only new, uncached ones).
//
// setdiff_kernel: one wavefront per pair. Slots whose block left the
//   selection are freed; each selected block that is not cached takes a free
//   slot (lowest first, in ascending block order) and becomes a copy-list
//   entry, unless it holds no token yet (a selection made one layer ahead,
//   before the append, includes the block the coming token opens: the
//   append creates it in its slot). O(k) work, a lane per selection entry
//   (two for k > 64) and per cache slot.
// gather_kernel: copies each listed 32 KiB block from the host store to its
//   cache slot, reading host memory through its device alias; one
//   workgroup per list entry.
// gather_wg_kernel: the same copies by a fixed number of workgroups that
//   loop over the entries (SparDA's persistent copy kernel with a workgroup
//   budget, aliyun article, KV 预取的运行时实现), so a fetch running beside
//   compute on another stream holds only that many workgroup slots.
#include "nosa_internal.h"

namespace nosa {
namespace {

__global__ __launch_bounds__(64) void setdiff_kernel(
    Dims d, nosa_state st, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ n_sel, int32_t *__restrict__ phys,
    int32_t *__restrict__ n_miss, int2 *__restrict__ list) {
  extern __shared__ __align__(16) uint32_t sel_bits[];   // [elig_words]
  __shared__ int bos_new[kMaxK + 1];
  __shared__ int free_list[kMaxK + 1];
  const int p = blockIdx.x, l = threadIdx.x;
  const int slots = d.k + 1;
  int32_t *sob = st.slot_of_block + (size_t)p * d.NB_max;
  int32_t *bos = st.block_of_slot + (size_t)p * slots;

  for (int i = l; i < d.elig_words; i += 64) sel_bits[i] = 0u;
  __syncthreads();
  const int ns = max(0, min(n_sel[p], d.k));
  const int L = st.seq_len[p / d.Hkv];          // blocks at or past it hold no token
  // lane l holds selection entries l and l + 64 (k <= 128)
  constexpr int kPer = kMaxK / 64;
  int blk[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = l + 64 * r;
    blk[r] = e < ns ? sel[(size_t)p * d.k + e] : -1;
    if (blk[r] >= d.NB_max) {
      atomicOr(st.status, NOSA_STATUS_BAD_SEL);
      blk[r] = -1;
    }
    if (blk[r] >= 0) atomicOr(&sel_bits[blk[r] >> 5], 1u << (blk[r] & 31));
  }
  __syncthreads();

  // slots: keep those holding a selected block, free the rest
  int n_free = 0;
  for (int base = 0; base < slots; base += 64) {
    const int s = base + l;
    int hb = -1;
    bool is_free = false;
    if (s < slots) {
      hb = bos[s];
      const bool keep = hb >= 0 && hb < d.NB_max && ((sel_bits[hb >> 5] >> (hb & 31)) & 1u);
      if (!keep) {
        if (hb >= 0 && hb < d.NB_max) sob[hb] = -1;     // evicted
        hb = -1;
        is_free = true;
      }
      bos_new[s] = hb;
    }
    const unsigned long long fm = __ballot(is_free);
    if (is_free) free_list[n_free + __popcll(fm & ((1ull << l) - 1ull))] = s;
    n_free += __popcll(fm);
  }
  __syncthreads();

  // misses take free slots in order (entry order = ascending block order);
  // those that hold tokens are listed for copying
  int n_missed = 0, n_copy = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = l + 64 * r;
    int slot = blk[r] >= 0 ? sob[blk[r]] : -1;
    const bool miss = blk[r] >= 0 && slot < 0;
    const unsigned long long mm = __ballot(miss);
    const int rank = n_missed + __popcll(mm & ((1ull << l) - 1ull));
    const bool copy = miss && rank < n_free && blk[r] * kBlock < L;
    const unsigned long long cm = __ballot(copy);
    const int crank = n_copy + __popcll(cm & ((1ull << l) - 1ull));
    if (miss) {
      slot = rank < n_free ? free_list[rank] : -1;
      if (slot >= 0) {
        bos_new[slot] = blk[r];
        sob[blk[r]] = slot;
        if (copy) list[(size_t)p * d.k + crank] = make_int2(blk[r], slot);
      } else {
        atomicOr(st.status, NOSA_STATUS_BAD_SEL);
      }
    }
    n_missed += __popcll(mm);
    n_copy += __popcll(cm);
    if (e < d.k) phys[(size_t)p * d.k + e] = e < ns ? slot : -1;
  }
  __syncthreads();
  for (int s = l; s < slots; s += 64) bos[s] = bos_new[s];
  if (l == 0) n_miss[p] = n_copy;
}

// grid (k, P), block 256: entry r of pair p, if it exists.
__global__ __launch_bounds__(256) void gather_kernel(
    Dims d, const uint16_t *__restrict__ host, uint16_t *__restrict__ cache,
    const int32_t *__restrict__ n_miss, const int2 *__restrict__ list) {
  const int r = blockIdx.x, p = blockIdx.y;
  if (r >= n_miss[p]) return;
  const int2 e = list[(size_t)p * d.k + r];
  const uint4 *src = reinterpret_cast<const uint4 *>(
      host + ((size_t)p * d.NB_kv + e.x) * kBlockElems);
  uint4 *dst = reinterpret_cast<uint4 *>(cache + ((size_t)p * (d.k + 1) + e.y) * kBlockElems);
  constexpr int kVec = kBlockElems * 2 / 16;   // 2048 uint4 per block
  uint4 v[kVec / 256];
#pragma unroll
  for (int j = 0; j < kVec / 256; ++j) v[j] = src[threadIdx.x + 256 * j];
#pragma unroll
  for (int j = 0; j < kVec / 256; ++j) dst[threadIdx.x + 256 * j] = v[j];
}

// grid (n_wg), block 256: workgroup i copies list entries i, i + n_wg, ...
// in entry-major order (entry r of every pair before entry r + 1), up to
// the largest copy count over the pairs; each block moves in pieces of
// VPT * 4 KiB, so a workgroup has at most that much host data in flight.
template <int VPT>
__global__ __launch_bounds__(256) void gather_wg_kernel(
    Dims d, const uint16_t *__restrict__ host, uint16_t *__restrict__ cache,
    const int32_t *__restrict__ n_miss, const int2 *__restrict__ list) {
  __shared__ int red[4];
  int m = 0;
  for (int i = threadIdx.x; i < d.P; i += 256) m = max(m, n_miss[i]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = max(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const int mx = min(max(max(red[0], red[1]), max(red[2], red[3])), d.k);
  const int total = mx * d.P;
  constexpr int kVec = kBlockElems * 2 / 16;   // 2048 uint4 per block
  for (int task = blockIdx.x; task < total; task += gridDim.x) {   // uniform
    const int r = task / d.P, p = task - r * d.P;
    if (r >= n_miss[p]) continue;
    const int2 e = list[(size_t)p * d.k + r];
    const uint4 *src = reinterpret_cast<const uint4 *>(
        host + ((size_t)p * d.NB_kv + e.x) * kBlockElems);
    uint4 *dst = reinterpret_cast<uint4 *>(cache + ((size_t)p * (d.k + 1) + e.y) * kBlockElems);
#pragma unroll
    for (int j0 = 0; j0 < kVec / 256; j0 += VPT) {
      uint4 v[VPT];
#pragma unroll
      for (int j = 0; j < VPT; ++j) v[j] = src[threadIdx.x + 256 * (j0 + j)];
#pragma unroll
      for (int j = 0; j < VPT; ++j) dst[threadIdx.x + 256 * (j0 + j)] = v[j];
    }
  }
}

// grid (n_wg), block 256: a plain copy through the gather's load path
// (16 bytes per thread and load, a workgroup moving 32 KiB per round like
// one block), for measuring the host link.
__global__ __launch_bounds__(256) void link_copy_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, size_t n16) {
  constexpr int kPer = 8;
  const size_t step = (size_t)gridDim.x * 256 * kPer;
  for (size_t base = (size_t)blockIdx.x * 256 * kPer; base < n16; base += step) {
    uint4 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const size_t i = base + threadIdx.x + 256 * j;
      if (i < n16) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const size_t i = base + threadIdx.x + 256 * j;
      if (i < n16) dst[i] = v[j];
    }
  }
}

// grid (n_wg), block 256: a plain streaming read, folded by XOR into one
// 16-byte word per thread (so the loads cannot be dropped), for measuring
// how fast the chip streams HBM with no other work. Workgroup i reads its
// own contiguous span of the buffer (as a decode wave reads its blocks),
// 4 KiB per round of 16-byte non-temporal loads (the policy of the decode's
// KV stream), 8 rounds in flight per thread.
typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4 *__restrict__ src,
                                                       size_t n16, uint4 *__restrict__ sink) {
  constexpr int kPer = 8;
  constexpr size_t kWindow = size_t(1) << 26;   // 16-byte words per buffer window (1 GiB)
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  u32x4n acc = {0u, 0u, 0u, 0u};
  for (size_t w0 = lo; w0 < hi; w0 += kWindow) {
    const uint32_t n = (uint32_t)(hi - w0 < kWindow ? hi - w0 : kWindow);   // words in the window
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4 *>(src + w0), (short)0, (int)(n * 16u), 0x00020000);
    uint32_t i = threadIdx.x;
    for (; i + (kPer - 1) * 256 < n; i += kPer * 256) {
      u32x4n v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (i + j * 256) * 16, 0, 2);   // nt
#pragma unroll
      for (int j = 0; j < kPer; ++j) acc ^= v[j];
    }
    for (; i < n; i += 256) acc ^= __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, 2);
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = make_uint4(acc[0], acc[1], acc[2], acc[3]);
}

// Resident KV: every selected block already sits in the device pool at its
// own index, so phys = sel and nothing moves. grid (P), block 64.
__global__ __launch_bounds__(64) void resident_phys_kernel(
    Dims d, const int32_t *__restrict__ sel, int32_t *__restrict__ phys,
    int32_t *__restrict__ n_miss) {
  const int p = blockIdx.x;
  for (int i = threadIdx.x; i < d.k; i += 64) phys[(size_t)p * d.k + i] = sel[(size_t)p * d.k + i];
  if (threadIdx.x == 0) n_miss[p] = 0;
}

}  // namespace

FetchLayout fetch_layout(const Dims &d) {
  FetchLayout f;
  f.list_off = 0;
  f.bytes = (((size_t)d.P * d.k * sizeof(int2)) + 255) & ~(size_t)255;
  return f;
}

hipError_t launch_link_copy(const void *src, void *dst, size_t bytes, int n_wg,
                            hipStream_t s) {
  link_copy_kernel<<<dim3(n_wg), 256, 0, s>>>(static_cast<const uint4 *>(src),
                                              static_cast<uint4 *>(dst), bytes / 16);
  return hipGetLastError();
}

hipError_t launch_hbm_read(const void *src, size_t bytes, int n_wg, void *sink, hipStream_t s) {
  hbm_read_kernel<<<dim3(n_wg), 256, 0, s>>>(static_cast<const uint4 *>(src), bytes / 16,
                                             static_cast<uint4 *>(sink));
  return hipGetLastError();
}

hipError_t launch_fetch(const Dims &d, const nosa_state &st, const int32_t *sel,
                        const int32_t *n_sel, int32_t *phys, int32_t *n_miss,
                        void *ws, const FetchLayout &lay, hipStream_t s, int n_wg) {
  if (!d.offload) {
    resident_phys_kernel<<<dim3(d.P), 64, 0, s>>>(d, sel, phys, n_miss);
    return hipGetLastError();
  }
  int2 *list = reinterpret_cast<int2 *>(static_cast<char *>(ws) + lay.list_off);
  setdiff_kernel<<<dim3(d.P), 64, (size_t)d.elig_words * sizeof(uint32_t), s>>>(
      d, st, sel, n_sel, phys, n_miss, list);
  if (n_wg > 0) {
    const int vpt = tuning(NOSA_TUNE_GATHER_VPT) ? tuning(NOSA_TUNE_GATHER_VPT) : 8;
    if (vpt == 1)
      gather_wg_kernel<1><<<dim3(n_wg), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
    else if (vpt == 2)
      gather_wg_kernel<2><<<dim3(n_wg), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
    else if (vpt == 4)
      gather_wg_kernel<4><<<dim3(n_wg), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
    else
      gather_wg_kernel<8><<<dim3(n_wg), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
  } else
    gather_kernel<<<dim3(d.k, d.P), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
  return hipGetLastError();
}

}  // namespace nosa
