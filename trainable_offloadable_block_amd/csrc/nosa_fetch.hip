// Delta fetch for offloaded KV (aiwiki "NOSA", NOSI: the inference system:
// a set-difference kernel between the previous and current selection so only
// changed blocks move, and a kernel that reads pinned host memory directly;
// SparDA article on aliyun, KV 预取的运行时实现: the GPU keeps the previous
// step's top-k blocks per layer and fetches only new, uncached ones).
//
// setdiff_kernel: one wavefront per pair. Slots whose block left the
//   selection are freed; each selected block that is not cached takes a free
//   slot (lowest first, in ascending block order) and becomes a copy-list
//   entry. O(k) work, a lane per selection entry (two for k > 64) and per
//   cache slot.
// gather_kernel: copies each listed 32 KiB block from the host store to its
//   cache slot, reading host memory through its device alias.
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

  // misses take free slots in order (entry order = ascending block order)
  int n_missed = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = l + 64 * r;
    int slot = blk[r] >= 0 ? sob[blk[r]] : -1;
    const bool miss = blk[r] >= 0 && slot < 0;
    const unsigned long long mm = __ballot(miss);
    const int rank = n_missed + __popcll(mm & ((1ull << l) - 1ull));
    if (miss) {
      slot = rank < n_free ? free_list[rank] : -1;
      if (slot >= 0) {
        bos_new[slot] = blk[r];
        sob[blk[r]] = slot;
        list[(size_t)p * d.k + rank] = make_int2(blk[r], slot);
      } else {
        atomicOr(st.status, NOSA_STATUS_BAD_SEL);
      }
    }
    n_missed += __popcll(mm);
    if (e < d.k) phys[(size_t)p * d.k + e] = e < ns ? slot : -1;
  }
  __syncthreads();
  for (int s = l; s < slots; s += 64) bos[s] = bos_new[s];
  if (l == 0) n_miss[p] = min(n_missed, n_free);
}

// grid (k, P), block 256: entry r of pair p, if it exists.
__global__ __launch_bounds__(256) void gather_kernel(
    Dims d, const uint16_t *__restrict__ host, uint16_t *__restrict__ cache,
    const int32_t *__restrict__ n_miss, const int2 *__restrict__ list) {
  const int r = blockIdx.x, p = blockIdx.y;
  if (r >= n_miss[p]) return;
  const int2 e = list[(size_t)p * d.k + r];
  const uint4 *src = reinterpret_cast<const uint4 *>(
      host + ((size_t)p * d.NB_max + e.x) * kBlockElems);
  uint4 *dst = reinterpret_cast<uint4 *>(cache + ((size_t)p * (d.k + 1) + e.y) * kBlockElems);
  constexpr int kVec = kBlockElems * 2 / 16;   // 2048 uint4 per block
  uint4 v[kVec / 256];
#pragma unroll
  for (int j = 0; j < kVec / 256; ++j) v[j] = src[threadIdx.x + 256 * j];
#pragma unroll
  for (int j = 0; j < kVec / 256; ++j) dst[threadIdx.x + 256 * j] = v[j];
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

hipError_t launch_fetch(const Dims &d, const nosa_state &st, const int32_t *sel,
                        const int32_t *n_sel, int32_t *phys, int32_t *n_miss,
                        void *ws, const FetchLayout &lay, hipStream_t s) {
  if (!d.offload) {
    resident_phys_kernel<<<dim3(d.P), 64, 0, s>>>(d, sel, phys, n_miss);
    return hipGetLastError();
  }
  int2 *list = reinterpret_cast<int2 *>(static_cast<char *>(ws) + lay.list_off);
  setdiff_kernel<<<dim3(d.P), 64, (size_t)d.elig_words * sizeof(uint32_t), s>>>(
      d, st, sel, n_sel, phys, n_miss, list);
  gather_kernel<<<dim3(d.k, d.P), 256, 0, s>>>(d, st.kv_host, st.kv_dev, n_miss, list);
  return hipGetLastError();
}

}  // namespace nosa
