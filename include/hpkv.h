/*
 * hpkv — block-paged KV cache hot path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libhpkv.so. Plain pointers and sizes only.
 *
 * Data model ("Block-Paged KV Cache", Hurray format documentation, section
 * "The three buffers"):
 *   page pool    K and V each [num_pages, page_size, num_kv_heads, head_dim],
 *                row-major, fully packed, one layer. A "slot" is one token row
 *                of the pool: slot = page * page_size + offset_in_page, and the
 *                row holds num_kv_heads * head_dim elements.
 *   block_table  physical page id of every logical page, all sequences
 *                concatenated (CSR); element type u32 or u64 (index_type).
 *   seq_ptr      num_seqs + 1 offsets into block_table, same element type;
 *                sequence s owns block_table[seq_ptr[s] .. seq_ptr[s+1]).
 * Token t of sequence s lives in slot
 *   block_table[seq_ptr[s] + t / page_size] * page_size + t % page_size
 * ("Block-Paged KV Cache", section "Element lookup through the block table";
 * "Paged KV Cache · AI infra interview lesson", section "Walk the Shapes
 * First"). Two table entries may name the same page (shared prefixes); reads
 * through aliased entries see the same bytes.
 *
 * Conventions for every entry point:
 *   - Return value: HPKV_OK (0) or a negative hpkv_status. Argument checks run
 *     on the host before any HIP call; on error nothing is launched and no
 *     output is touched.
 *   - Device entry points take device pointers owned by the caller and enqueue
 *     work on `stream` (a hipStream_t; NULL means the null stream). They
 *     return once the work is enqueued; they never allocate, free or
 *     synchronise. Launch failures are reported as HPKV_ERR_HIP.
 *   - Host entry points (validate, element offset) take host pointers and
 *     never touch the GPU.
 *   - Contents of device index buffers are not checked by the device entry
 *     points (call hpkv_validate_index_buffers on host copies first, as the
 *     Hurray page recommends before shipping a descriptor). The kernels still
 *     never read or write outside the buffers described by the sizes passed;
 *     malformed contents give the documented fallback results below.
 */
#ifndef HPKV_H_
#define HPKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HPKV_OK = 0,
  HPKV_ERR_NULL = -1,          /* a required pointer is NULL */
  HPKV_ERR_INVALID_ARG = -2,   /* a size or enum argument is out of range */
  HPKV_ERR_INVALID_INDEX = -3, /* index buffer contents break an invariant (host checks) */
  HPKV_ERR_UNSUPPORTED = -4,   /* valid but not implemented (e.g. head_dim shape) */
  HPKV_ERR_HIP = -5,           /* the HIP runtime reported an error at launch */
  HPKV_ERR_WORKSPACE = -6,     /* workspace missing or too small */
  HPKV_ERR_SCRATCH_LIMIT = -7  /* needs more scratch than the no-allocation decode holds */
} hpkv_status;

/* Element type of block_table and seq_ptr ("Block-Paged KV Cache", section
 * "Building a descriptor": 32-bit indices, or 64-bit for huge pools). */
typedef enum { HPKV_INDEX_U32 = 0, HPKV_INDEX_U64 = 1 } hpkv_index_type;

/* Element type of q, out, new K/V rows and the page pools. */
typedef enum { HPKV_F32 = 0, HPKV_F16 = 1, HPKV_BF16 = 2 } hpkv_dtype;

/* Element type of quantized page pools, one byte per element: two's-complement
 * int8, or OCP 8-bit float E4M3 in its "fn" variant (bias 7, largest finite
 * magnitude 448, no infinity, NaN = 0x7f / 0xff). */
typedef enum { HPKV_KV_I8 = 3, HPKV_KV_FP8_E4M3 = 4 } hpkv_kv_type;

/* Static description of a status code (never NULL). */
const char* hpkv_status_string(int status);

/* ---------------------------------------------------------------------------
 * hpkv_validate_index_buffers  (host)
 *
 * Checks the storage invariants of "Block-Paged KV Cache", section
 * "Validating the storage invariants": seq_ptr[0] == 0, seq_ptr
 * non-decreasing, seq_ptr[num_seqs] == block_table_len, and every
 * block_table entry < num_pages. num_seqs == 0 with seq_ptr == {0} is valid.
 * When context_lens (host, num_seqs entries) is non-NULL, each length must
 * also satisfy 0 <= ctx <= (seq_ptr[s+1] - seq_ptr[s]) * page_size.
 *   seq_ptr      host, num_seqs + 1 entries of index_type
 *   block_table  host, block_table_len entries (may be NULL if len == 0)
 * Returns HPKV_OK, HPKV_ERR_INVALID_INDEX on a broken invariant, or an
 * argument error.
 * ------------------------------------------------------------------------- */
int hpkv_validate_index_buffers(int index_type, uint64_t num_pages, uint64_t num_seqs,
                                const void* seq_ptr, const void* block_table,
                                uint64_t block_table_len, const int32_t* context_lens,
                                uint32_t page_size);

/* ---------------------------------------------------------------------------
 * hpkv_element_offset  (host)
 *
 * Flat page-pool offset (in elements) of logical element
 * (sequence s, token t, head h, dim d):
 *   ((block_table[seq_ptr[s] + t/page_size] * page_size + t%page_size)
 *      * num_heads + h) * head_dim + d
 * ("Block-Paged KV Cache", section "Element lookup through the block table").
 * Host pointers. Writes *flat_out and returns HPKV_OK, or returns
 * HPKV_ERR_INVALID_INDEX when s, the token's page, h, d or the page id is out
 * of range.
 * ------------------------------------------------------------------------- */
int hpkv_element_offset(int index_type, uint64_t s, uint64_t t, uint32_t h, uint32_t d,
                        uint32_t page_size, uint64_t num_pages, uint32_t num_heads,
                        uint32_t head_dim, const void* block_table, uint64_t block_table_len,
                        const void* seq_ptr, uint64_t num_seqs, uint64_t* flat_out);

/* ---------------------------------------------------------------------------
 * hpkv_validate_shape  (host)
 *
 * The logical tensor of a block-paged cache is rank 3,
 * [total_tokens, num_heads, head_dim] ("Block-Paged KV Cache", section
 * "Building a descriptor"). Returns HPKV_OK for rank 3 with non-zero heads and
 * dims, HPKV_ERR_INVALID_ARG otherwise. dims: host array of `rank` entries.
 * ------------------------------------------------------------------------- */
int hpkv_validate_shape(uint32_t rank, const uint64_t* dims);

/* ---------------------------------------------------------------------------
 * hpkv_slot_mapping  (device)
 *
 * Pool slot of every new token ("Paged KV Cache · AI infra interview lesson",
 * section "Step 1: slot_mapping and store_kvcache", and "Walk the Shapes
 * First"): new-token row i of sequence s, cu_new[s] <= i < cu_new[s+1], is at
 * position p = start_pos[s] + (i - cu_new[s]) and gets
 *   slots[i] = block_table[seq_ptr[s] + p/page_size] * page_size + p%page_size.
 * A chunk may start part-way into a page (prefix hit, second half of a
 * chunked prefill). A position whose page is not in the sequence's slice,
 * whose block_table index is >= block_table_len, or whose page id is
 * >= num_pages (outside the pool: the storage invariant of "Block-Paged KV
 * Cache", section "Validating index buffers", does not hold there) gets -1,
 * the skip value, so a store never writes outside the pool.
 *   block_table  device, block_table_len entries of index_type
 *   seq_ptr      device, num_seqs + 1 entries of index_type
 *   start_pos    device int32 [num_seqs]
 *   cu_new       device int64 [num_seqs + 1], cu_new[0] == 0,
 *                non-decreasing, cu_new[num_seqs] == num_new
 *   slots        device int64 [num_new], written
 * num_seqs == 0 or num_new == 0 launches nothing.
 * ------------------------------------------------------------------------- */
int hpkv_slot_mapping(int index_type, const void* block_table, uint64_t block_table_len,
                      const void* seq_ptr, uint32_t num_seqs, uint32_t page_size,
                      uint64_t num_pages, const int32_t* start_pos, const int64_t* cu_new, uint64_t num_new,
                      int64_t* slots, void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_store_kvcache  (device)
 *
 * Scatter of freshly computed rows into the pools ("Paged KV Cache · AI infra
 * interview lesson", section "Step 1: slot_mapping and store_kvcache"): for
 * every i < num_tokens with slots[i] != -1, K row i (num_kv_heads*head_dim
 * elements of key) is copied bit for bit to slot slots[i] of k_cache, and
 * likewise value -> v_cache. Slots < 0 or >= num_pages*page_size are skipped.
 * Two rows with the same slot race (undefined which one lands); callers must
 * not alias writable slots.
 *   key, value        device [num_tokens, num_kv_heads, head_dim] of dtype
 *   k_cache, v_cache  device [num_pages, page_size, num_kv_heads, head_dim]
 *   slots             device int64 [num_tokens]
 * num_tokens == 0 launches nothing.
 * ------------------------------------------------------------------------- */
int hpkv_store_kvcache(int dtype, const void* key, const void* value, void* k_cache,
                       void* v_cache, const int64_t* slots, uint64_t num_tokens,
                       uint32_t page_size, uint64_t num_pages, uint32_t num_kv_heads,
                       uint32_t head_dim, void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode_workspace_size  (host)
 *
 * Bytes of device workspace hpkv_paged_attention_decode needs for a batch of
 * num_seqs sequences no longer than max_context_len tokens: the split-context
 * partials (one fp32 (max, sum) pair and one fp32 head_dim vector per
 * sequence, query head and context partition), then the dispatch order of the
 * (sequence, partition) pairs (one uint32 each) and one byte per pair for
 * hpkv_paged_attention_decode_shared, counted with the smallest
 * partition the library uses, so it is enough for every num_kv_heads and for
 * the quantized decode. 0 when every sequence fits one partition (no
 * workspace is then read or written) and on invalid arguments.
 * ------------------------------------------------------------------------- */
size_t hpkv_paged_attention_decode_workspace_size(int dtype, uint32_t num_seqs,
                                                  uint32_t num_q_heads, uint32_t head_dim,
                                                  uint32_t page_size, uint32_t max_context_len);

/* Context tokens covered by one split-context partition of
 * hpkv_paged_attention_decode (and of the _step and _reduce entry points) for
 * this call shape: 2048 when the batch still gives at least 1024 workgroups
 * with partitions that long, else 1024 when it gives at least 256 (one per
 * CU), else 512.
 * Exposed for accounting and tests. 0 on invalid arguments. */
uint32_t hpkv_paged_attention_decode_partition_tokens(int dtype, uint32_t num_seqs,
                                                      uint32_t num_q_heads,
                                                      uint32_t num_kv_heads, uint32_t head_dim,
                                                      uint32_t page_size,
                                                      uint32_t max_context_len);

/* The same for hpkv_paged_attention_decode_quant (kv_type HPKV_KV_I8 or
 * HPKV_KV_FP8_E4M3): the same thresholds, among the partitions whose pages fit
 * the kernels' per-page table (at most 520 pages: 2048 tokens needs pages of 4
 * or more tokens, 1024 of 2 or more); 2048-token partitions only where the
 * matrix-core kernel runs (16-bit dtype, GQA groups of 4 or more, head_dim 32,
 * 64 or 128). 0 on invalid arguments. */
uint32_t hpkv_paged_attention_decode_quant_partition_tokens(int dtype, int kv_type,
                                                            uint32_t num_seqs,
                                                            uint32_t num_q_heads,
                                                            uint32_t num_kv_heads,
                                                            uint32_t head_dim, uint32_t page_size,
                                                            uint32_t max_context_len);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode  (device)
 *
 * Single-query paged decode attention ("Paged KV Cache · AI infra interview
 * lesson", section "Step 2: paged_attention_decode"; the cached step
 * Attn(q_t, [K_1..t], [V_1..t]) of "LLM Inference Engineering & Economics",
 * Chapter 2, section "What the KV cache actually stores"). For every
 * sequence s and query head h, with n = context_lens[s] and KV head
 * g = h / (num_q_heads / num_kv_heads) (GQA, consecutive grouping):
 *   z_t   = scale * dot(q[s,h,:], K[token t of s, g, :])      t < n
 *   out[s,h,:] = sum_t softmax(z)_t * V[token t of s, g, :]
 * K/V rows are gathered through the block table; only the first
 * ceil(n/page_size) pages of the slice and only rows t < n are read (rows past
 * the context in the last page are never loaded, so their contents, NaN
 * included, do not matter). n == 0 gives zeros.
 * Arithmetic: fp32 dot products and online softmax, fp32 accumulation, one
 * rounding (nearest-even) to dtype at the end; with one exception. For f16
 * and bf16 with head_dim in {32, 64, 128} and num_q_heads / num_kv_heads a
 * multiple of 4, the scores and P.V run on the matrix cores: there each
 * softmax weight exp(z_t - running max) is rounded (nearest-even) to dtype
 * before it multiplies V, and the softmax denominator sums those rounded
 * weights, so the output is a convex combination of V rows with weights
 * accurate to dtype's precision (about 2^-9 relative for bf16). Everything
 * else (dot products, maxima, sums, the accumulator, the split merge) stays
 * fp32.
 *   q, out            device [num_seqs, num_q_heads, head_dim] of dtype
 *   k_cache, v_cache  device pools of dtype
 *   block_table, seq_ptr  device, as above
 *   context_lens      device int32 [num_seqs]
 *   max_context_len   host upper bound of context_lens (sizes the launch)
 *   workspace         device, >= hpkv_paged_attention_decode_workspace_size
 *                     bytes (contents need no initialisation)
 * Requirements: q, k_cache, v_cache and workspace 16-byte aligned
 * (HPKV_ERR_INVALID_ARG otherwise); num_q_heads % num_kv_heads == 0;
 * head_dim in {8, 16, 32, 64, 128, 256} (any dtype),
 * otherwise HPKV_ERR_UNSUPPORTED. When the matrix-core kernel serves two KV
 * heads per workgroup (16-bit dtype, GQA groups of 4 or more, even
 * num_kv_heads, large batches), num_pages * page_size must not exceed 2^32
 * (its row table holds 32-bit pool slots; such a pool takes at least 512 GiB):
 * HPKV_ERR_UNSUPPORTED otherwise. The partition grid (head tiles x partitions x
 * num_seqs workgroups) must stay below 2^24 workgroups (HPKV_ERR_UNSUPPORTED).
 * Malformed contents (caller error): a sequence with n < 0,
 * n > max_context_len, n beyond its slice, or a page id >= num_pages in the
 * pages it reads, gets NaN in all its outputs.
 * Enqueued: a one-workgroup ordering pass that lists the (sequence,
 * partition) pairs longest partition first in the workspace (skipped when the
 * grid has at most 512 workgroups, or no workspace is needed), the
 * split-context partition pass, which takes its work in that order so the
 * launch does not end on a few long partitions, then the log-sum-exp reduce
 * (skipped per sequence when one partition covers it). Results do not depend
 * on the order.
 * ------------------------------------------------------------------------- */
int hpkv_paged_attention_decode(int dtype, int index_type, const void* q, const void* k_cache,
                                const void* v_cache, const void* block_table,
                                uint64_t block_table_len, const void* seq_ptr,
                                const int32_t* context_lens, uint32_t num_seqs,
                                uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                                uint32_t page_size, uint64_t num_pages, float scale,
                                uint32_t max_context_len, void* workspace, size_t workspace_bytes,
                                void* out, void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode_noalloc  (device)
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * hpkv_paged_attention_decode, same kernels and results, without the
 * workspace arguments. The workspace is a fixed array inside the library,
 * hpkv_paged_attention_decode_noalloc_max_workspace() bytes (128 MiB) per GPU,
 * held by each GPU the library runs on until the process ends; its device
 * address is looked up on the first call on each device. The call allocates
 * nothing. A batch whose hpkv_paged_attention_decode_workspace_size exceeds
 * that maximum returns HPKV_ERR_SCRATCH_LIMIT before any GPU work. Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, or threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. Every other argument,
 * requirement and error is that of hpkv_paged_attention_decode.
 * ------------------------------------------------------------------------- */
size_t hpkv_paged_attention_decode_noalloc_max_workspace(void);
int hpkv_paged_attention_decode_noalloc(int dtype, int index_type, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const void* block_table, uint64_t block_table_len,
                                        const void* seq_ptr, const int32_t* context_lens,
                                        uint32_t num_seqs, uint32_t num_q_heads,
                                        uint32_t num_kv_heads, uint32_t head_dim,
                                        uint32_t page_size, uint64_t num_pages, float scale,
                                        uint32_t max_context_len, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode_shared  (device)
 *
 * hpkv_paged_attention_decode for batches whose sequences alias pages, as
 * shared prefixes do ("Block-Paged KV Cache", "Element lookup through the
 * block table": aliased tables resolve to the same offsets; "Paged KV Cache ·
 * AI infra interview lesson", "Step 5": prefix pages shared by reference).
 * Same arguments, requirements, errors and results, bit for bit: every output
 * equals what hpkv_paged_attention_decode gives on the same inputs with every
 * aliased page replaced by a private copy. The difference is the work: on the
 * matrix-core path (bf16/f16, head_dim in {32, 64, 128}, num_q_heads /
 * num_kv_heads a multiple of 4 and at most 8 per tile) a detection pass
 * compares the block tables, and a context partition that is full and covers
 * the same page ids for consecutive sequences of an aligned block of
 * 32 / (query heads per tile) sequences is read once, by one workgroup, for
 * all of them. Elsewhere, and for batches that fit one partition per
 * sequence, it behaves as hpkv_paged_attention_decode. The detection pass and
 * the ordering pass run even when nothing is shared (a few microseconds).
 * ------------------------------------------------------------------------- */
int hpkv_paged_attention_decode_shared(int dtype, int index_type, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const void* block_table, uint64_t block_table_len,
                                       const void* seq_ptr, const int32_t* context_lens,
                                       uint32_t num_seqs, uint32_t num_q_heads,
                                       uint32_t num_kv_heads, uint32_t head_dim,
                                       uint32_t page_size, uint64_t num_pages, float scale,
                                       uint32_t max_context_len, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream);

/* The two passes of hpkv_paged_attention_decode, separately: the partition
 * pass (the ordering kernel, then the partition kernel, which writes `out` for
 * sequences covered by one partition and partials for the rest) and the
 * reduce (merges the partials into `out`). Calling them in this
 * order on one stream with the same arguments is equivalent to
 * hpkv_paged_attention_decode. Used to time the kernels one by one. */
int hpkv_paged_attention_decode_partitions(int dtype, int index_type, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const void* block_table, uint64_t block_table_len,
                                           const void* seq_ptr, const int32_t* context_lens,
                                           uint32_t num_seqs, uint32_t num_q_heads,
                                           uint32_t num_kv_heads, uint32_t head_dim,
                                           uint32_t page_size, uint64_t num_pages, float scale,
                                           uint32_t max_context_len, void* workspace,
                                           size_t workspace_bytes, void* out, void* stream);
int hpkv_paged_attention_decode_reduce(int dtype, const int32_t* context_lens, uint32_t num_seqs,
                                       uint32_t num_q_heads, uint32_t num_kv_heads,
                                       uint32_t head_dim, uint32_t page_size,
                                       uint32_t max_context_len, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode_step  (device)
 *
 * One fused decode step: for every sequence s with n = context_lens[s] >= 1
 * the freshly computed K and V rows of its newest token (position n-1, the
 * decode slot of "Paged KV Cache · AI infra interview lesson", sections
 * "Walk the Shapes First" and "Common Pitfalls") are written into the pools
 * at slot block_table[seq_ptr[s] + (n-1)/page_size]*page_size + (n-1)%page_size,
 * and decode attention then runs over all n tokens, exactly as
 * hpkv_slot_mapping (start_pos = n-1, one token per sequence) +
 * hpkv_store_kvcache + hpkv_paged_attention_decode, in the decode's own
 * launches (the row is stored by the workgroup that reads it).
 *   new_key, new_value  device [num_seqs, num_kv_heads, head_dim] of dtype,
 *                       16-byte aligned
 *   slots_out           device int64 [num_seqs] or NULL: the slot each row went
 *                       to, -1 for n == 0 and for malformed sequences
 * Every other argument, requirement and error is that of
 * hpkv_paged_attention_decode (k_cache and v_cache are written). A sequence
 * the decode reports as malformed (NaN output) gets no row written.
 * ------------------------------------------------------------------------- */
int hpkv_paged_attention_decode_step(int dtype, int index_type, const void* q,
                                     const void* new_key, const void* new_value, void* k_cache,
                                     void* v_cache, const void* block_table,
                                     uint64_t block_table_len, const void* seq_ptr,
                                     const int32_t* context_lens, uint32_t num_seqs,
                                     uint32_t num_q_heads, uint32_t num_kv_heads,
                                     uint32_t head_dim, uint32_t page_size, uint64_t num_pages,
                                     float scale, uint32_t max_context_len, int64_t* slots_out,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_prefill  (device)
 *
 * Causal attention of a prefill chunk over the paged cache. A chunk may start
 * part-way into a page, after a prefix hit or an earlier chunk ("Paged KV
 * Cache · AI infra interview lesson", section "Step 1: slot_mapping and
 * store_kvcache"); its queries read K/V through the block table as in
 * section "Step 2: paged_attention_decode", including pages aliased across
 * sequences ("Block-Paged KV Cache", section "Element lookup through the
 * block table"). Sequence s owns query rows i = cu_q[s] .. cu_q[s+1]-1 at
 * positions p = q_start[s] + (i - cu_q[s]); for query head h and KV head
 * g = h / (num_q_heads / num_kv_heads)
 *   out[i,h,:] = sum_{t <= p} softmax_t(scale * q[i,h,:] . K[t,g,:]) V[t,g,:].
 * The chunk's own K/V rows must already be in the pools (hpkv_slot_mapping +
 * hpkv_store_kvcache first).
 *   q, out        device [num_q_tokens, num_q_heads, head_dim] of dtype,
 *                 16-byte aligned; out is written for every query row of
 *                 every sequence (caller-owned, not aliasing q or the pools)
 *   k_cache, v_cache, block_table, seq_ptr, page_size, num_pages: as for
 *                 hpkv_paged_attention_decode (read only)
 *   q_start       device int32 [num_seqs]
 *   cu_q          device int64 [num_seqs + 1], non-decreasing, cu_q[0] = 0,
 *                 cu_q[num_seqs] = num_q_tokens
 *   max_q_len     >= every chunk length cu_q[s+1] - cu_q[s] (sizes the grid);
 *                 must be >= 1 when num_q_tokens > 0
 *   stream        hipStream_t or NULL; the call only enqueues (asynchronous)
 * Supported: dtype bf16 or f16, head_dim in {32, 64, 128, 256}, and
 * num_q_heads / num_kv_heads at most 128 (the rows of one workgroup),
 * num_pages * page_size below 2^32 (pool rows are kept in 32 bits) and fewer
 * than 2^31 workgroups (ceil(min(max_q_len, num_q_tokens) * group / 128)
 * position blocks x num_kv_heads x num_seqs); otherwise
 * HPKV_ERR_UNSUPPORTED. Argument errors (NULL pointers, zero sizes, heads not
 * divisible, NaN scale, misaligned buffers) return before any GPU work.
 * Malformed contents (caller error): a sequence whose chunk is longer than
 * max_q_len, has negative q_start or bad cu_q entries, or runs past its slice
 * gets NaN in all its rows; rows whose keys include a page id >= num_pages
 * get NaN. Nothing is read or written out of bounds.
 * One kernel is enqueued; no workspace is needed.
 * ------------------------------------------------------------------------- */
int hpkv_paged_attention_prefill(int dtype, int index_type, const void* q, const void* k_cache,
                                 const void* v_cache, const void* block_table,
                                 uint64_t block_table_len, const void* seq_ptr,
                                 const int32_t* q_start, const int64_t* cu_q, uint32_t num_seqs,
                                 uint64_t num_q_tokens, uint32_t num_q_heads,
                                 uint32_t num_kv_heads, uint32_t head_dim, uint32_t page_size,
                                 uint64_t num_pages, float scale, uint32_t max_q_len, void* out,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * Quantized page pools.
 *
 * "Block-Paged KV Cache", section "Quantization compatibility": KV caches are
 * often int8/fp8, and per-block-affine quantization is allowed only along the
 * paged axis with block_size == page_size, so the scales belong to a physical
 * page slot and a page shared by several sequences carries its own. The
 * dequantization formula is not given there; this library takes the affine
 * reading: each page slot holds, per KV head, an fp32 scale and zero point
 * for K and another pair for V, and a code c stands for
 *   scale * (value(c) - zero)
 * with value(c) the int8 integer or the E4M3 number.
 *   k_scale, k_zero, v_scale, v_zero   device fp32 [num_pages, num_kv_heads]
 *   k_cache, v_cache                   device [num_pages, page_size,
 *                                      num_kv_heads, head_dim] of kv_type
 * Scales must be finite and non-zero; zero points finite.
 * ------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------
 * hpkv_store_kvcache_quant  (device)
 *
 * hpkv_store_kvcache into quantized pools: for every i < num_tokens whose slot
 * is in [0, num_pages*page_size), element x of K row i (KV head g) is written
 * as the code nearest to t = x / k_scale[page, g] + k_zero[page, g] (page =
 * slot / page_size; the division rounded to nearest fp32, then the add), ties
 * to even, saturating at the type's range (int8 [-128, 127], E4M3 +-448); NaN
 * gives 0 (int8) or 0x7f (E4M3). Likewise V with v_scale / v_zero. Other
 * slots are skipped; repeated slots race.
 *   key, value   device [num_tokens, num_kv_heads, head_dim] of dtype,
 *                16-byte aligned
 *   head_dim     a multiple of 8 (else HPKV_ERR_UNSUPPORTED)
 * ------------------------------------------------------------------------- */
int hpkv_store_kvcache_quant(int dtype, int kv_type, const void* key, const void* value,
                             void* k_cache, void* v_cache, const float* k_scale,
                             const float* k_zero, const float* v_scale, const float* v_zero,
                             const int64_t* slots, uint64_t num_tokens, uint32_t page_size,
                             uint64_t num_pages, uint32_t num_kv_heads, uint32_t head_dim,
                             void* stream);

/* ---------------------------------------------------------------------------
 * hpkv_paged_attention_decode_quant  (device)
 *
 * hpkv_paged_attention_decode over quantized pools: every K/V element is
 * taken as scale * (value(code) - zero) of its page slot and KV head. q and
 * out keep dtype (f32, f16 or bf16); arithmetic is fp32 (the page
 * scale multiplies each score, the V scale each weight, and the zero points
 * enter as one correction per row), except that on the matrix-core path
 * (f16/bf16 q, head_dim in {32, 64, 128}, num_q_heads / num_kv_heads a
 * multiple of 4) each weight times its V scale is rounded (nearest-even) to
 * dtype before it multiplies the V codes, and the V zero-point correction
 * uses those rounded products; the denominator sums the unrounded fp32
 * weights. Off the matrix cores, int8 K codes against an f16 or bf16 q with an
 * even num_q_heads / num_kv_heads enter the scores as exact f16 products
 * (code + 1152 times q, a bf16 q first scaled per head by the power of two
 * that puts its largest magnitude in [2^14, 2^15); elements under 2^-31 of
 * that magnitude then fall below f16's normal range and are truncated),
 * summed in fp32; with fp8 codes, an f16 or bf16 q and num_q_heads /
 * num_kv_heads even but not a multiple of 4 there (tiles of two query heads),
 * each weight times its V scale is rounded (nearest-even) to bf16
 * before it multiplies the V codes, the V zero-point correction uses those
 * rounded products and the denominator sums the unrounded fp32 weights.
 * The workspace, its size function
 * (hpkv_paged_attention_decode_workspace_size with the same dtype), the
 * tail masking, the malformed-input NaN results and the argument errors are
 * those of hpkv_paged_attention_decode. Requirements: head_dim in
 * {16, 32, 64, 128, 256}; q, k_cache, v_cache and workspace 16-byte aligned;
 * num_pages * num_kv_heads < 2^32.
 * ------------------------------------------------------------------------- */
int hpkv_paged_attention_decode_quant(int dtype, int kv_type, int index_type, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* k_scale, const float* k_zero,
                                      const float* v_scale, const float* v_zero,
                                      const void* block_table, uint64_t block_table_len,
                                      const void* seq_ptr, const int32_t* context_lens,
                                      uint32_t num_seqs, uint32_t num_q_heads,
                                      uint32_t num_kv_heads, uint32_t head_dim,
                                      uint32_t page_size, uint64_t num_pages, float scale,
                                      uint32_t max_context_len, void* workspace,
                                      size_t workspace_bytes, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Host block manager (host; no GPU work).
 *
 * Owner of the physical pages that block tables name ("Paged KV Cache · AI
 * infra interview lesson", sections "Walk the Shapes First" and "Step 5:
 * BlockManager: ref counts and chained-hash prefix caching"; "LLM Inference
 * Engineering & Economics", Chapter 2, sections "PagedAttention separates
 * logical space from physical space", "Prefix reuse is another optimization"
 * and "Deterministic evals for this layer"):
 *   - a pool of num_pages pages of page_size tokens and a free list;
 *   - a sequence gets a new page exactly when its length becomes
 *     len % page_size == 1;
 *   - every page counts the block tables that hold it and returns to the free
 *     list only when the last one releases it;
 *   - a full page is registered under XXH64 of its page_size token ids (int32,
 *     little-endian) seeded with the hash of the previous page of the same
 *     sequence (0 for the first), so the hash covers the whole prefix; a new
 *     sequence reuses the leading full pages whose hash and tokens match (the
 *     partially filled last page is never shared, so no writable page has two
 *     owners);
 *   - free pages are reused first-freed first; a freed page stays in the
 *     prefix cache until it is handed out for other content.
 * Not thread-safe: one caller at a time per manager.
 * Errors: HPKV_ERR_NULL (missing pointer), HPKV_ERR_INVALID_ARG (unknown or
 * duplicate seq_id, bad enum), HPKV_ERR_INVALID_INDEX (out of free pages; the
 * state is unchanged), HPKV_ERR_WORKSPACE (export capacity too small; the
 * needed length is still reported).
 * ------------------------------------------------------------------------- */
typedef struct hpkv_block_manager hpkv_block_manager;

/* New manager over pages 0 .. num_pages-1, all free; NULL if a size is 0 or
 * memory runs out. */
hpkv_block_manager* hpkv_bm_create(uint64_t num_pages, uint32_t page_size);
void hpkv_bm_destroy(hpkv_block_manager* bm);

/* Admits sequence seq_id with its first num_tokens token ids (a prompt, host
 * int32 array): reuses cached leading full pages, takes fresh pages for the
 * rest and registers every full page. *cached_tokens (may be NULL) receives
 * the number of prompt tokens whose pages were reused (a multiple of
 * page_size), i.e. whose K/V need not be computed again. */
int hpkv_bm_admit(hpkv_block_manager* bm, uint64_t seq_id, const int32_t* token_ids,
                  uint64_t num_tokens, uint64_t* cached_tokens);

/* Appends one token; takes a fresh page when the new length is
 * len % page_size == 1. *slot (may be NULL) receives the pool slot of the new
 * token, position len-1 (the decode slot of "Common Pitfalls"). */
int hpkv_bm_append(hpkv_block_manager* bm, uint64_t seq_id, int32_t token_id, int64_t* slot);

/* Drops the sequence's references (its pages, last first). */
int hpkv_bm_release(hpkv_block_manager* bm, uint64_t seq_id);

/* Free and allocated page counts (free + allocated = num_pages), live
 * sequences and pages registered in the prefix cache; any pointer may be NULL. */
int hpkv_bm_stats(const hpkv_block_manager* bm, uint64_t* free_pages, uint64_t* allocated_pages,
                  uint64_t* live_sequences, uint64_t* cached_pages);

/* Writes the CSR tables of the listed sequences, in that order, as the
 * device entry points take them: block_table (capacity entries of
 * index_type), seq_ptr (num_seqs + 1 entries) and context_lens (int32
 * [num_seqs], may be NULL), all host memory. *block_table_len receives the
 * entries needed. */
int hpkv_bm_export(const hpkv_block_manager* bm, const uint64_t* seq_ids, uint32_t num_seqs,
                   int index_type, void* block_table, uint64_t capacity, void* seq_ptr,
                   int32_t* context_lens, uint64_t* block_table_len);

/* Checks the accounting invariants: every page's reference count equals the
 * number of live tables that hold it; a page is free exactly when that count
 * is 0 and the free list holds each free page; free + allocated = pool; a
 * partially filled (writable) page has one owner and is not shared through the
 * prefix cache; every prefix-cache entry names a full page with that hash.
 * HPKV_OK or HPKV_ERR_INVALID_INDEX. */
int hpkv_bm_check(const hpkv_block_manager* bm);

/* XXH64 of len bytes with the given seed (the page hash above). */
uint64_t hpkv_xxh64(const void* data, uint64_t len, uint64_t seed);

/* ---------------------------------------------------------------------------
 * hpkv_read_ceiling  (device; measurement)
 *
 * Reads `bytes` of device memory in the access pattern of the decode gather
 * and nothing else, to measure the HBM read ceiling the decode kernels are
 * held against (decode attention reads every context row of K and V once:
 * "Paged KV Cache · AI infra interview lesson", section "Step 2:
 * paged_attention_decode"). The buffer is viewed as rows of stride_bytes,
 * each split into stride_bytes / row_bytes columns of row_bytes; one
 * workgroup reads one column of rows_per_workgroup consecutive rows, with
 * 16-byte non-temporal loads as the decode kernels issue them. row_bytes ==
 * stride_bytes is a plain streaming read; row_bytes 256 at stride 8192 is the
 * (page row, KV head) pattern of a 32-KV-head, d = 128, bf16 pool. Only the
 * first floor(bytes / stride_bytes) rows are read. sink (device, 4 bytes) is
 * written only in the practically impossible case that a lane's data folds to
 * one fixed word; its contents mean nothing.
 * Requirements: buf 16-byte aligned; row_bytes a power of two in [16, 4096];
 * stride_bytes a multiple of row_bytes; rows_per_workgroup >= 1
 * (HPKV_ERR_INVALID_ARG otherwise; HPKV_ERR_NULL for NULL pointers).
 * ------------------------------------------------------------------------- */
int hpkv_read_ceiling(const void* buf, uint64_t bytes, uint32_t row_bytes,
                      uint64_t stride_bytes, uint32_t rows_per_workgroup, uint32_t* sink,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HPKV_H_ */
