// Slot mapping and KV scatter ("store") kernels for gfx950.
//
// Slot rule ("Paged KV Cache · AI infra interview lesson", sections "Walk the
// Shapes First" and "Step 1: slot_mapping and store_kvcache"; block table in
// the CSR form of "Block-Paged KV Cache", section "The three buffers"):
//   slot(s, p) = block_table[seq_ptr[s] + p / page_size] * page_size + p % page_size
// Store: every new-token row with a slot other than -1 is copied bit for bit
// into that pool row of K and of V.
#include "hpkv_device.h"

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
    uint32_t num_seqs, uint32_t page_size, uint64_t num_pages,
    const int32_t* __restrict__ start_pos, const int64_t* __restrict__ cu_new, uint64_t num_new,
    int64_t* __restrict__ slots) {
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
        if (phys < num_pages) slot = int64_t(phys * page_size + uint64_t(p) % page_size);
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

// ---------------------------------------------------------------------------
// Quantized store ("Block-Paged KV Cache", section "Quantization
// compatibility": per-block-affine with one block per page, so each page slot
// carries its own scale and zero point per KV head). Element x of a new row is
// written as the code nearest to t = x / scale + zero (fp32 division rounded
// to nearest, then the add), ties to even, saturating: int8 in [-128, 127];
// OCP fp8 E4M3 ("e4m3fn": bias 7, largest finite 448, no infinity) at +-448.
// NaN gives 0 (int8) or the NaN code 0x7f (fp8).
// ---------------------------------------------------------------------------

__device__ inline uint32_t quant_i8(float t) {
  if (t != t) return 0u;
  const float r = fminf(fmaxf(rintf(t), -128.0f), 127.0f);  // rintf: ties to even
  return uint32_t(int32_t(r)) & 0xffu;
}

__device__ inline uint32_t quant_fp8_e4m3(float t) {
  if (t != t) return 0x7fu;
  const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
  const float a = fabsf(t);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7eu;  // saturate
  } else if (a < 0.015625f) {
    code = uint32_t(rintf(a * 512.0f));  // subnormal quantum 2^-9 (8 -> 2^-6, code 0x08)
  } else {
    const int e = int((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a in [2^e, 2^(e+1))
    const float m = __uint_as_float(__float_as_uint(a) & 0x807fffffu | 0x3f800000u);  // [1, 2)
    const uint32_t f = uint32_t(rintf((m - 1.0f) * 8.0f));  // 0..8, exact product, ties to even
    code = (uint32_t(e + 7) << 3) + f;  // f == 8 carries into the exponent
  }
  return sign | code;
}

template <int DT, int QT>
__device__ inline uint32_t quant_code(float t) {
  if constexpr (QT == kI8) {
    return quant_i8(t);
  } else {
    return quant_fp8_e4m3(t);
  }
}

// One workgroup per new row; each thread turns 8 elements of one KV head of the
// row (K and V) into 8 codes.
template <int DT, int QT>
__global__ __launch_bounds__(kStoreThreads) void store_quant_kernel(
    const void* __restrict__ key, const void* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ k_zero, const float* __restrict__ v_scale,
    const float* __restrict__ v_zero, const int64_t* __restrict__ slots, uint64_t num_tokens,
    uint32_t page_size, int64_t num_slots, uint32_t num_kv_heads, uint32_t head_dim) {
  constexpr int EB = Elem<DT>::bytes;
  const uint32_t groups = num_kv_heads * head_dim / 8;  // 8-element groups per row
  for (uint64_t rowi = blockIdx.x; rowi < num_tokens; rowi += gridDim.x) {
    const int64_t slot = slots[rowi];
    if (slot < 0 || slot >= num_slots) continue;
    const uint64_t page = uint64_t(slot) / page_size;
    for (uint32_t gi = threadIdx.x; gi < groups; gi += kStoreThreads) {
      const uint32_t g = gi * 8 / head_dim;
      const uint64_t f = page * num_kv_heads + g;
      const uint64_t src = (rowi * num_kv_heads * head_dim + uint64_t(gi) * 8) * EB;
      float xk[8], xv[8];
#pragma unroll
      for (int h = 0; h < 8 * EB / 16; ++h) {
        float tk[16 / EB], tv[16 / EB];
        widen16<DT>(*reinterpret_cast<const u32x4*>(static_cast<const char*>(key) + src + 16 * h), tk);
        widen16<DT>(*reinterpret_cast<const u32x4*>(static_cast<const char*>(value) + src + 16 * h), tv);
#pragma unroll
        for (int e = 0; e < 16 / EB; ++e) {
          xk[h * (16 / EB) + e] = tk[e];
          xv[h * (16 / EB) + e] = tv[e];
        }
      }
      const float ks = k_scale[f], kz = k_zero[f], vs = v_scale[f], vz = v_zero[f];
      uint32_t ck[2] = {0u, 0u}, cv[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ck[e / 4] |= quant_code<DT, QT>(__fdiv_rn(xk[e], ks) + kz) << (8 * (e % 4));
        cv[e / 4] |= quant_code<DT, QT>(__fdiv_rn(xv[e], vs) + vz) << (8 * (e % 4));
      }
      const uint64_t dst = uint64_t(slot) * num_kv_heads * head_dim + uint64_t(gi) * 8;
      *reinterpret_cast<uint2*>(k_cache + dst) = make_uint2(ck[0], ck[1]);
      *reinterpret_cast<uint2*>(v_cache + dst) = make_uint2(cv[0], cv[1]);
    }
  }
}

}  // namespace

hipError_t launch_slot_mapping(bool idx64, const void* block_table, uint64_t block_table_len,
                               const void* seq_ptr, uint32_t num_seqs, uint32_t page_size,
                               uint64_t num_pages, const int32_t* start_pos, const int64_t* cu_new, uint64_t num_new,
                               int64_t* slots, hipStream_t stream) {
  const uint64_t blocks = (num_new + kSlotThreads - 1) / kSlotThreads;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  if (idx64) {
    hipLaunchKernelGGL(slot_mapping_kernel<uint64_t>, dim3(uint32_t(blocks)), dim3(kSlotThreads),
                       0, stream, static_cast<const uint64_t*>(block_table), block_table_len,
                       static_cast<const uint64_t*>(seq_ptr), num_seqs, page_size, num_pages, start_pos,
                       cu_new, num_new, slots);
  } else {
    hipLaunchKernelGGL(slot_mapping_kernel<uint32_t>, dim3(uint32_t(blocks)), dim3(kSlotThreads),
                       0, stream, static_cast<const uint32_t*>(block_table), block_table_len,
                       static_cast<const uint32_t*>(seq_ptr), num_seqs, page_size, num_pages, start_pos,
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

template <int DT>
hipError_t launch_store_quant_dt(int kv_type, const void* key, const void* value, void* k_cache,
                                 void* v_cache, const float* ks, const float* kz,
                                 const float* vs, const float* vz, const int64_t* slots,
                                 uint64_t num_tokens, uint32_t page_size, int64_t num_slots,
                                 uint32_t num_kv_heads, uint32_t head_dim, hipStream_t stream) {
  const uint32_t blocks = uint32_t(num_tokens < (1u << 20) ? num_tokens : (1u << 20));
  uint8_t* kc = static_cast<uint8_t*>(k_cache);
  uint8_t* vc = static_cast<uint8_t*>(v_cache);
  if (kv_type == kI8) {
    hipLaunchKernelGGL((store_quant_kernel<DT, kI8>), dim3(blocks), dim3(kStoreThreads), 0,
                       stream, key, value, kc, vc, ks, kz, vs, vz, slots, num_tokens, page_size,
                       num_slots, num_kv_heads, head_dim);
  } else if (kv_type == kFP8) {
    hipLaunchKernelGGL((store_quant_kernel<DT, kFP8>), dim3(blocks), dim3(kStoreThreads), 0,
                       stream, key, value, kc, vc, ks, kz, vs, vz, slots, num_tokens, page_size,
                       num_slots, num_kv_heads, head_dim);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_store_quant(int dtype, int kv_type, const void* key, const void* value,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* k_zero, const float* v_scale, const float* v_zero,
                              const int64_t* slots, uint64_t num_tokens, uint32_t page_size,
                              uint64_t num_pages, uint32_t num_kv_heads, uint32_t head_dim,
                              hipStream_t stream) {
  const int64_t num_slots = int64_t(num_pages * page_size);
  switch (dtype) {
    case kF32:
      return launch_store_quant_dt<kF32>(kv_type, key, value, k_cache, v_cache, k_scale, k_zero,
                                         v_scale, v_zero, slots, num_tokens, page_size, num_slots,
                                         num_kv_heads, head_dim, stream);
    case kF16:
      return launch_store_quant_dt<kF16>(kv_type, key, value, k_cache, v_cache, k_scale, k_zero,
                                         v_scale, v_zero, slots, num_tokens, page_size, num_slots,
                                         num_kv_heads, head_dim, stream);
    case kBF16:
      return launch_store_quant_dt<kBF16>(kv_type, key, value, k_cache, v_cache, k_scale, k_zero,
                                          v_scale, v_zero, slots, num_tokens, page_size,
                                          num_slots, num_kv_heads, head_dim, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace hpkv
