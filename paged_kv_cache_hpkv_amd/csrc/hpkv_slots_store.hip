// Slot mapping and KV scatter ("store") kernels for gfx950.
//
// Slot rule ("Paged KV Cache · AI infra interview lesson", sections "Walk the
// Shapes First" and "Step 1: slot_mapping and store_kvcache"; block table in
// the CSR form of "Block-Paged KV Cache", section "The three buffers"):
//   slot(s, p) = block_table[seq_ptr[s] + p / page_size] * page_size + p % page_size
// Store: every new-token row with a slot other than -1 is copied bit for bit
// into that pool row of K and of V.
#include "hpkv_internal.h"

namespace hpkv {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kStoreThreads = 256;

// cu_new entries a slot-mapping workgroup stages in LDS for its search.
constexpr uint32_t kSlotLdsSeqs = 4096;

// One thread per new token. The owning sequence is found by binary search over
// cu_new (the largest s with cu_new[s] <= i), which keeps the launch balanced
// whatever the mix of chunk lengths. Batches of up to kSlotLdsSeqs sequences
// search a copy of cu_new staged in LDS by the workgroup (one coalesced read
// instead of a chain of dependent global reads).
template <typename Idx>
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const Idx* __restrict__ block_table, uint64_t block_table_len, const Idx* __restrict__ seq_ptr,
    uint32_t num_seqs, uint32_t page_size, const int32_t* __restrict__ start_pos,
    const int64_t* __restrict__ cu_new, uint64_t num_new, int64_t* __restrict__ slots) {
  __shared__ int64_t s_cu[kSlotLdsSeqs + 1];
  const bool staged = num_seqs <= kSlotLdsSeqs;
  if (staged) {
    for (uint32_t k = threadIdx.x; k <= num_seqs; k += kSlotThreads) s_cu[k] = cu_new[k];
    __syncthreads();
  }
  const int64_t* cu = staged ? s_cu : cu_new;
  const uint64_t i = uint64_t(blockIdx.x) * kSlotThreads + threadIdx.x;
  if (i >= num_new) return;
  // upper bound of i in cu[1 .. num_seqs]
  uint32_t lo = 1, hi = num_seqs + 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if (cu[mid] <= int64_t(i)) {
      lo = mid + 1;
    } else {
      hi = mid;
    }
  }
  const uint32_t s = lo - 1;
  int64_t slot = -1;
  if (s < num_seqs && cu[s] <= int64_t(i)) {
    const int64_t p = int64_t(start_pos[s]) + (int64_t(i) - cu[s]);
    const uint64_t first = seq_ptr[s];
    const uint64_t last = seq_ptr[s + 1];
    if (p >= 0 && first <= last && last <= block_table_len) {
      const uint64_t page_in_seq = uint64_t(p) / page_size;
      if (page_in_seq < last - first) {
        const uint64_t phys = block_table[first + page_in_seq];
        slot = int64_t(phys * page_size + uint64_t(p) % page_size);
      }
    }
  }
  slots[i] = slot;
}

// One workgroup per new-token row (grid-strided); each thread copies
// `Chunk`-sized pieces of the row for K and V. The row is read while its slot
// is still in flight (the source address does not depend on it); rows whose
// slot is -1, negative or past the pool are skipped.
template <typename Chunk>
__global__ __launch_bounds__(kStoreThreads) void store_kernel(
    const Chunk* __restrict__ key, const Chunk* __restrict__ value, Chunk* __restrict__ k_cache,
    Chunk* __restrict__ v_cache, const int64_t* __restrict__ slots, uint64_t num_tokens,
    uint64_t row_chunks, int64_t num_slots) {
  for (uint64_t row = blockIdx.x; row < num_tokens; row += gridDim.x) {
    const int64_t slot = slots[row];
    const Chunk* ksrc = key + row * row_chunks;
    const Chunk* vsrc = value + row * row_chunks;
    for (uint64_t c = threadIdx.x; c < row_chunks; c += kStoreThreads) {
      const Chunk kv = ksrc[c];
      const Chunk vv = vsrc[c];
      if (slot >= 0 && slot < num_slots) {
        k_cache[uint64_t(slot) * row_chunks + c] = kv;
        v_cache[uint64_t(slot) * row_chunks + c] = vv;
      }
    }
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

}  // namespace

hipError_t launch_slot_mapping(bool idx64, const void* block_table, uint64_t block_table_len,
                               const void* seq_ptr, uint32_t num_seqs, uint32_t page_size,
                               const int32_t* start_pos, const int64_t* cu_new, uint64_t num_new,
                               int64_t* slots, hipStream_t stream) {
  const uint64_t blocks = (num_new + kSlotThreads - 1) / kSlotThreads;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  if (idx64) {
    hipLaunchKernelGGL(slot_mapping_kernel<uint64_t>, dim3(uint32_t(blocks)), dim3(kSlotThreads),
                       0, stream, static_cast<const uint64_t*>(block_table), block_table_len,
                       static_cast<const uint64_t*>(seq_ptr), num_seqs, page_size, start_pos,
                       cu_new, num_new, slots);
  } else {
    hipLaunchKernelGGL(slot_mapping_kernel<uint32_t>, dim3(uint32_t(blocks)), dim3(kSlotThreads),
                       0, stream, static_cast<const uint32_t*>(block_table), block_table_len,
                       static_cast<const uint32_t*>(seq_ptr), num_seqs, page_size, start_pos,
                       cu_new, num_new, slots);
  }
  return hipGetLastError();
}

hipError_t launch_store(int chunk_bytes, const void* key, const void* value, void* k_cache,
                        void* v_cache, const int64_t* slots, uint64_t num_tokens,
                        uint64_t row_chunks, int64_t num_slots, hipStream_t stream) {
  const uint32_t blocks = uint32_t(num_tokens < (1u << 20) ? num_tokens : (1u << 20));
  switch (chunk_bytes) {
    case 16:
      hipLaunchKernelGGL(store_kernel<u32x4>, dim3(blocks), dim3(kStoreThreads), 0, stream,
                         static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
                         static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slots,
                         num_tokens, row_chunks, num_slots);
      break;
    case 4:
      hipLaunchKernelGGL(store_kernel<uint32_t>, dim3(blocks), dim3(kStoreThreads), 0, stream,
                         static_cast<const uint32_t*>(key), static_cast<const uint32_t*>(value),
                         static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache), slots,
                         num_tokens, row_chunks, num_slots);
      break;
    case 2:
      hipLaunchKernelGGL(store_kernel<uint16_t>, dim3(blocks), dim3(kStoreThreads), 0, stream,
                         static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                         static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), slots,
                         num_tokens, row_chunks, num_slots);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hpkv
