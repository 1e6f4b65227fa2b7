// Internal interface between the host entry points (hpkv_api.cpp) and the
// gfx950 kernels (*.hip). Not installed; the public ABI is include/hpkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hpkv {

// Element storage types, same numbering as hpkv_dtype.
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };
// Quantized pool element types, same numbering as hpkv_kv_type.
enum : int { kI8 = 3, kFP8 = 4 };

inline int dtype_bytes(int dt) { return dt == kF32 ? 4 : 2; }

// Split-context partitions, in context tokens, as sizes of the decode kernels'
// LDS row tables: the quantized kernels and the matrix-core kernel with one KV
// head per workgroup hold kMaxPartTokens; the VALU kernel and the matrix-core
// kernel with two KV heads per workgroup hold kLongPartTokens (the latter as
// 32-bit pool slots). Partitions of kWidePartTokens and kLongPartTokens run on
// those two kernels.
constexpr uint32_t kMaxPartTokens = 512;
constexpr uint32_t kWidePartTokens = 1024;
constexpr uint32_t kLongPartTokens = 2048;
// The quantized kernels keep their row table per page: a partition may touch at
// most this many pages (P tokens starting anywhere in a page of bs tokens touch
// at most (P + bs - 2) / bs + 1): 512 tokens of 1-token pages, 1024 of 2-token
// pages, 2048 of pages of 4 or more.
constexpr uint32_t kQuantTablePages = 520;
inline uint32_t partition_pages_max(uint32_t part_tokens, uint32_t page_size) {
  return (part_tokens + page_size - 2) / page_size + 1;
}

// Division by a runtime divisor 1 <= d < 2^31 for numerators n < 2^31:
// n / d == (n * mul) >> shift with shift = 31 + ceil(log2 d) and
// mul = ceil(2^shift / d) (< 2^32). Exact because the rounding excess of mul
// times n stays below 2^shift.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint32_t shift = 31 + l;
  const unsigned __int128 num = (unsigned __int128)1 << shift;
  const uint64_t mul = uint64_t((num + d - 1) / d);
  return FastDiv{uint32_t(mul), shift};
}

struct DecodeKernelArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const void* block_table;
  const void* seq_ptr;
  const int32_t* context_lens;
  float* ws_o;       // [B, Hq, max_parts, head_dim] unnormalised partial outputs
  float2* ws_ml;     // [B, Hq, max_parts] (running max in log2 units, sum of weights)
  uint64_t block_table_len;
  uint64_t num_pages;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t page_size;
  uint32_t group;       // num_q_heads / num_kv_heads
  uint32_t head_tiles;  // (num_kv_heads / kv_per_wg) * (group / heads per workgroup)
  uint32_t kv_per_wg;   // adjacent KV heads per workgroup (> 1: whole GQA groups)
  uint32_t max_parts;
  uint32_t part_tokens;
  uint32_t max_context_len;
  FastDiv page_div;
  float scale_log2;     // scale * log2(e): scores are kept in base-2 units
  int idx64;            // block_table / seq_ptr hold u64 (else u32)
  // Fused decode step (all null for a plain decode): the row of each
  // sequence's last context token is written into the pools before it is read.
  const void* new_k;    // [B, Hkv, d] K rows of the appended tokens
  const void* new_v;    // [B, Hkv, d] V rows
  int64_t* slots_out;   // [B] pool slot each row went to (-1: none), may be null
  // Quantized pools (kv_type kI8 / kFP8, 1-byte elements; dtype is then the
  // type of q and out): fp32 [num_pages, Hkv] scale and zero point of each page
  // slot and KV head, for K and for V. Null for 16/32-bit pools.
  int kv_type;
  const float* k_scale;
  const float* k_zero;
  const float* v_scale;
  const float* v_zero;
  // Dispatch order of the (sequence, partition) pairs, longest partitions
  // first: [num_seqs * max_parts] pair indices s + num_seqs * part, written by
  // the ordering pass ahead of the partition pass. Null: plain partition-major
  // order.
  uint32_t* order;
  // Shared partitions (hpkv_paged_attention_decode_shared on the matrix cores):
  // sequences are grouped in aligned blocks of share_block (1: no sharing), and
  // share_flags[s + num_seqs * part] = 1 when partition `part` of sequence s is
  // full and covers the same page ids as that of sequence s - 1 in its block.
  // The ordering pass then writes such a follower as no work, and the entry of
  // the run's first sequence carries the run's length in its top bits.
  uint32_t share_block;
  uint8_t* share_flags;
};

struct ReduceKernelArgs {
  const int32_t* context_lens;
  const float* ws_o;
  const float2* ws_ml;
  void* out;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t head_dim;
  uint32_t max_parts;
  uint32_t part_tokens;
  uint32_t max_context_len;
};

struct PrefillKernelArgs {
  const void* q;             // [num_q_tokens, Hq, d]
  const void* k_cache;
  const void* v_cache;
  void* out;                 // [num_q_tokens, Hq, d]
  const void* block_table;
  const void* seq_ptr;
  const int32_t* q_start;    // [B] position of each chunk's first query
  const int64_t* cu_q;       // [B+1] query rows of sequence s: cu_q[s] .. cu_q[s+1]-1
  uint64_t block_table_len;
  uint64_t num_pages;
  uint64_t num_q_tokens;
  uint32_t num_seqs;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t page_size;
  uint32_t group;            // num_q_heads / num_kv_heads
  uint32_t block_positions;  // chunk positions one workgroup covers
  uint32_t pos_blocks;       // workgroups per (sequence, KV head)
  uint32_t max_q_len;
  uint32_t num_work;         // num_seqs * num_kv_heads * pos_blocks
  FastDiv page_div;
  float scale_log2;
  int idx64;
};

// Rows (query position x query head pairs) one prefill workgroup covers.
uint32_t prefill_rows_per_workgroup(int dtype, uint32_t head_dim);
bool prefill_head_dim_supported(int dtype, uint32_t head_dim);

hipError_t launch_prefill(int dtype, uint32_t head_dim, const PrefillKernelArgs& a,
                          uint32_t num_workgroups, hipStream_t stream);

// Query heads served by one decode workgroup for a GQA group of `group` heads
// (the matrix-core path takes up to 16 heads of a group at once).
uint32_t heads_per_workgroup(int dtype, uint32_t head_dim, uint32_t group);
// Whether the 16/32-bit decode of a shape runs on the matrix cores, and the
// same for quantized pools.
bool decode_on_matrix_cores(int dtype, uint32_t head_dim, uint32_t group);
bool decode_quant_on_matrix_cores(int dtype, uint32_t head_dim, uint32_t group);
// Most adjacent KV heads one decode workgroup may serve (whole GQA groups and
// an even number of KV heads only): two on the matrix cores; on the VALU kernel
// as many as make a token's row for the workgroup ~512 contiguous bytes, up to 4.
uint32_t kv_heads_per_workgroup(int dtype, uint32_t head_dim, uint32_t group,
                                uint32_t num_kv_heads);
// The same for quantized pools.
uint32_t heads_per_workgroup_quant(int dtype, uint32_t head_dim, uint32_t group);

hipError_t launch_decode_partitions_quant(int dtype, int kv_type, uint32_t head_dim,
                                          const DecodeKernelArgs& a, uint64_t num_workgroups,
                                          hipStream_t stream);

hipError_t launch_store_quant(int dtype, int kv_type, const void* key, const void* value,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* k_zero, const float* v_scale, const float* v_zero,
                              const int64_t* slots, uint64_t num_tokens, uint32_t page_size,
                              uint64_t num_pages, uint32_t num_kv_heads, uint32_t head_dim,
                              hipStream_t stream);

// Bytes of the fixed device scratch behind hpkv_paged_attention_decode_noalloc
// (per GPU), and the current device's address of it (looked up on first use).
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_read_ceiling(const void* buf, uint64_t bytes, uint32_t row_bytes,
                               uint64_t stride, uint32_t rows_per_wg, uint32_t* sink,
                               hipStream_t stream);

hipError_t launch_slot_mapping(bool idx64, const void* block_table, uint64_t block_table_len,
                               const void* seq_ptr, uint32_t num_seqs, uint32_t page_size,
                               uint64_t num_pages, const int32_t* start_pos, const int64_t* cu_new, uint64_t num_new,
                               int64_t* slots, hipStream_t stream);

hipError_t launch_store(int chunk_bytes, const void* key, const void* value, void* k_cache,
                        void* v_cache, const int64_t* slots, uint64_t num_tokens,
                        uint64_t row_chunks, int64_t num_slots, hipStream_t stream);

// Order-list entries of a shared run: pair index in the low bits, run length - 1
// above them.
constexpr uint32_t kRunShift = 29;
constexpr uint32_t kPairMask = (1u << kRunShift) - 1;

hipError_t launch_decode_partitions(int dtype, uint32_t head_dim, const DecodeKernelArgs& a,
                                    uint64_t num_workgroups, hipStream_t stream);

hipError_t launch_decode_reduce(int dtype, const ReduceKernelArgs& a, hipStream_t stream);

}  // namespace hpkv
