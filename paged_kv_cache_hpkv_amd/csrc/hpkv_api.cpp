// Host side of libhpkv.so: argument checks, host-only helpers and kernel
// launches behind the C ABI declared in include/hpkv.h. Every check runs
// before the first HIP call, so malformed calls fail without touching the GPU.
#include "hpkv.h"

#include <hip/hip_runtime.h>

#include "hpkv_internal.h"

namespace {

using hpkv::DecodeKernelArgs;
using hpkv::ReduceKernelArgs;

// Context tokens per split-context partition: 512 (kPartTokens), 1024 or 2048
// (hpkv::kWidePartTokens, hpkv::kLongPartTokens, where the kernel's row table
// holds that many and the batch still gives enough workgroups). The partials
// stay ~1-2 % of the KV bytes.
constexpr uint32_t kPartTokens = 512;
static_assert(kPartTokens <= hpkv::kMaxPartTokens, "partition larger than the LDS row table");
static_assert(kPartTokens <= hpkv::kWidePartTokens, "the workspace is sized for the smaller one");
// Fewest workgroups a coarser launch shape may leave: one per CU. Measured on
// MI355X, GQA 32/8 at 16 x 4096 tokens: 256 two-head workgroups with 1024-token
// partitions beat 1024 one-head workgroups (44 vs 47 us); at 1 x 4096 tokens,
// 64 one-head workgroups beat 16 two-head ones (13 vs 23 us).
constexpr uint64_t kMinWorkgroups = 256;
// 2048-token partitions halve the workgroups, and with them each workgroup's
// fixed costs (row table, merge), for long contexts; they need four times the
// workgroups of the other shapes so that the longest-first order still balances.
constexpr uint64_t kMinLongWorkgroups = 4 * kMinWorkgroups;
// Grids up to this many workgroups are resident on the 256 CUs at once (two
// per CU), so their dispatch order does not matter.
constexpr uint64_t kOrderMinWorkgroups = 512;

bool valid_dtype(int dt) { return dt == HPKV_F32 || dt == HPKV_F16 || dt == HPKV_BF16; }
bool valid_index(int it) { return it == HPKV_INDEX_U32 || it == HPKV_INDEX_U64; }

uint64_t read_index(int it, const void* p, uint64_t i) {
  return it == HPKV_INDEX_U64 ? static_cast<const uint64_t*>(p)[i]
                              : static_cast<const uint32_t*>(p)[i];
}

// head_dim * bytes must split into 16-byte lane chunks whose count is a power
// of two no larger than a wavefront, and head_dim must be a compiled size.
bool decode_head_dim_supported(int dtype, uint32_t head_dim) {
  switch (head_dim) {
    case 8: case 16: case 32: case 64: case 128: case 256: break;
    default: return false;
  }
  const uint32_t lanes = head_dim * uint32_t(hpkv::dtype_bytes(dtype)) / 16;
  return lanes >= 1 && lanes <= 64 && (lanes & (lanes - 1)) == 0;
}

// Quantized pools: 16 one-byte codes per lane chunk, a power-of-two number of
// lanes per row.
bool quant_head_dim_supported(uint32_t head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 ||
         head_dim == 256;
}

uint32_t max_parts_for(uint32_t max_context_len, uint32_t part_tokens) {
  return max_context_len == 0 ? 1u : (max_context_len + part_tokens - 1) / part_tokens;
}

// Launch shape of a decode call: query heads per workgroup (gt), adjacent KV
// heads per workgroup (hpw) and tokens per partition. Larger work units spread
// each workgroup's fixed costs (row table, first loads, merge) over more bytes
// (measured on MI355X: +8 % for the GQA batch with two KV heads and 1024-token
// partitions, +2-3 % for the VALU kernel with 1024-token partitions), but a
// small batch needs the finer ones to fill the GPU: the coarsest shape whose
// grid keeps kMinWorkgroups workgroups is taken, else the finest. Quantized
// pools keep 512-token partitions; their VALU kernel may serve two KV heads
// (a token's codes of one head are a single 128-byte line at d=128, and such
// rows stream markedly slower than two heads' 256 contiguous bytes).
struct DecodePlan {
  uint32_t gt, hpw, part_tokens;
};

DecodePlan plan_decode(int dtype, bool quant, uint32_t num_seqs, uint32_t num_q_heads,
                       uint32_t num_kv_heads, uint32_t head_dim, uint32_t page_size,
                       uint32_t max_context_len) {
  const uint32_t group = num_q_heads / num_kv_heads;
  DecodePlan c[6];  // candidate shapes, coarsest first
  int n = 0;
  if (quant) {
    // Partitions whose pages fit the kernels' per-page table. 2048 tokens only on the
    // matrix cores: the VALU kernel's two-wave workgroups (six per CU) are left too
    // few rounds by them (measured: qwen3 int8 0.506 ms at 1024, 0.588 at 2048;
    // quantized GQA on the matrix cores 0.222 at 1024, 0.209 at 2048).
    const bool mfma = hpkv::decode_quant_on_matrix_cores(dtype, head_dim, group);
    const uint32_t gt = hpkv::heads_per_workgroup_quant(dtype, head_dim, group);
    const uint32_t hpw = gt == group && num_kv_heads % 2 == 0 ? 2 : 1;
    for (uint32_t p : {hpkv::kLongPartTokens, hpkv::kWidePartTokens})
      if ((mfma || p != hpkv::kLongPartTokens) &&
          hpkv::partition_pages_max(p, page_size) <= hpkv::kQuantTablePages)
        c[n++] = {gt, hpw, p};
    c[n++] = {gt, hpw, kPartTokens};
    if (hpw > 1) c[n++] = {gt, 1, kPartTokens};
  } else if (hpkv::decode_on_matrix_cores(dtype, head_dim, group)) {
    const uint32_t gt = hpkv::heads_per_workgroup(dtype, head_dim, group);
    if (hpkv::kv_heads_per_workgroup(dtype, head_dim, group, num_kv_heads) > 1) {
      c[n++] = {gt, 2, hpkv::kLongPartTokens};
      c[n++] = {gt, 2, hpkv::kWidePartTokens};
      c[n++] = {gt, 2, kPartTokens};
    }
    c[n++] = {gt, 1, kPartTokens};
  } else {
    const uint32_t gt = hpkv::heads_per_workgroup(dtype, head_dim, group);
    const uint32_t hpw = hpkv::kv_heads_per_workgroup(dtype, head_dim, group, num_kv_heads);
    c[n++] = {gt, hpw, hpkv::kLongPartTokens};
    for (uint32_t h = hpw; h > 1; h /= 2) c[n++] = {gt, h, hpkv::kWidePartTokens};
    c[n++] = {gt, 1, hpkv::kWidePartTokens};
    c[n++] = {gt, 1, kPartTokens};
  }
  for (int i = 0; i + 1 < n; ++i) {
    const uint64_t grid = uint64_t(num_kv_heads / c[i].hpw) * (group / c[i].gt) * num_seqs *
                          max_parts_for(max_context_len, c[i].part_tokens);
    const uint64_t need =
        c[i].part_tokens == hpkv::kLongPartTokens ? kMinLongWorkgroups : kMinWorkgroups;
    if (grid >= need) return c[i];
  }
  return c[n - 1];
}

struct WorkspaceLayout {
  size_t ml_offset, o_offset, order_offset, flags_offset, bytes;
};

WorkspaceLayout workspace_layout(uint32_t num_seqs, uint32_t num_q_heads, uint32_t head_dim,
                                 uint32_t max_context_len, uint32_t part_tokens) {
  const uint64_t mp = max_parts_for(max_context_len, part_tokens);
  WorkspaceLayout w{0, 0, 0, 0, 0};
  if (mp <= 1) return w;  // every sequence fits one partition: no partials
  const uint64_t rows = uint64_t(num_seqs) * num_q_heads * mp;
  const uint64_t ml_bytes = (rows * sizeof(float2) + 255) & ~uint64_t(255);
  const uint64_t o_bytes = (rows * head_dim * sizeof(float) + 255) & ~uint64_t(255);
  const uint64_t order_bytes = (uint64_t(num_seqs) * mp * sizeof(uint32_t) + 255) & ~uint64_t(255);
  w.ml_offset = 0;
  w.o_offset = ml_bytes;
  w.order_offset = ml_bytes + o_bytes;          // one u32 per (sequence, partition)
  w.flags_offset = w.order_offset + order_bytes;  // then one byte per pair (shared runs)
  w.bytes = w.flags_offset + uint64_t(num_seqs) * mp;
  return w;
}

// Shared checks and argument packing of the decode entry points.
int prepare_decode(int dtype, int index_type, const void* q, const void* k_cache,
                   const void* v_cache, const void* block_table, uint64_t block_table_len,
                   const void* seq_ptr, const int32_t* context_lens, uint32_t num_seqs,
                   uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                   uint32_t page_size, uint64_t num_pages, float scale, uint32_t max_context_len,
                   void* workspace, size_t workspace_bytes, void* out, DecodeKernelArgs* a,
                   uint64_t* num_workgroups, int kv_type = -1, bool share = false) {
  if (!valid_dtype(dtype) || !valid_index(index_type)) return HPKV_ERR_INVALID_ARG;
  const bool quant = kv_type >= 0;
  if (quant && kv_type != HPKV_KV_I8 && kv_type != HPKV_KV_FP8_E4M3) return HPKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return HPKV_OK;
  if (!q || !k_cache || !v_cache || !seq_ptr || !context_lens || !out) return HPKV_ERR_NULL;
  if (block_table_len > 0 && !block_table) return HPKV_ERR_NULL;
  if (num_q_heads == 0 || num_kv_heads == 0 || head_dim == 0 || page_size == 0 ||
      num_pages == 0)
    return HPKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return HPKV_ERR_INVALID_ARG;
  if (page_size > 0x7fffffffu || max_context_len > 0x7fffffffu) return HPKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return HPKV_ERR_INVALID_ARG;  // NaN scale
  if (quant ? !quant_head_dim_supported(head_dim) : !decode_head_dim_supported(dtype, head_dim))
    return HPKV_ERR_UNSUPPORTED;
  if (quant && num_pages > 0xffffffffull / num_kv_heads) return HPKV_ERR_UNSUPPORTED;
  // q, K and V are read with 16-byte vector loads
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0)
    return HPKV_ERR_INVALID_ARG;
  const uint32_t group = num_q_heads / num_kv_heads;
  const DecodePlan plan = plan_decode(dtype, quant, num_seqs, num_q_heads, num_kv_heads,
                                      head_dim, page_size, max_context_len);
  const uint32_t hpw = plan.hpw, gt = plan.gt, part_tokens = plan.part_tokens;
  const WorkspaceLayout w =
      workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, part_tokens);
  if (w.bytes > 0 && (!workspace || workspace_bytes < w.bytes)) return HPKV_ERR_WORKSPACE;
  if (w.bytes > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return HPKV_ERR_INVALID_ARG;

  // the two-head matrix-core kernel keeps 32-bit pool slots in its row table; a
  // pool of more slots holds at least 2^32 * 256 bytes per K and V, beyond any one
  // GPU's memory
  if (!quant && hpw > 1 && hpkv::decode_on_matrix_cores(dtype, head_dim, group) &&
      num_pages > (uint64_t(1) << 32) / page_size)
    return HPKV_ERR_UNSUPPORTED;
  const uint32_t max_parts = max_parts_for(max_context_len, part_tokens);
  const uint64_t head_tiles = uint64_t(num_kv_heads / hpw) * (group / gt);
  const uint64_t nwg = head_tiles * max_parts * num_seqs;
  if (nwg > 0xffffffffull / 256) return HPKV_ERR_UNSUPPORTED;  // launch grid limit

  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->out = out;
  a->block_table = block_table;
  a->seq_ptr = seq_ptr;
  a->context_lens = context_lens;
  a->ws_ml = w.bytes ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + w.ml_offset)
                     : nullptr;
  a->ws_o = w.bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + w.o_offset)
                    : nullptr;
  a->block_table_len = block_table_len;
  a->num_pages = num_pages;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = num_kv_heads;
  a->page_size = page_size;
  a->group = group;
  a->head_tiles = uint32_t(head_tiles);
  a->kv_per_wg = hpw;
  a->max_parts = max_parts;
  a->part_tokens = part_tokens;
  a->max_context_len = max_context_len;
  a->page_div = hpkv::make_fastdiv(page_size);
  a->scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a->idx64 = index_type == HPKV_INDEX_U64;
  a->new_k = nullptr;
  a->new_v = nullptr;
  a->slots_out = nullptr;
  a->kv_type = quant ? kv_type : dtype;
  a->k_scale = a->k_zero = a->v_scale = a->v_zero = nullptr;
  // Longest-first dispatch pays when the grid is deeper than what the chip
  // holds at once; smaller grids keep the plain order and skip the pass.
  // Shared runs need the ordering pass (it drops the runs' followers), whatever the
  // grid: matrix-core tiles only, groups of at most 8 query heads per tile (runs of up
  // to 32/gt sequences: two blocks of 16 tile columns), and pair indices that leave the
  // run length room.
  const bool shared = share && !quant && w.bytes > 0 &&
                      hpkv::decode_on_matrix_cores(dtype, head_dim, group) && gt <= 8 &&
                      uint64_t(num_seqs) * max_parts <= hpkv::kPairMask;
  a->share_block = shared ? 32 / gt : 1;
  a->share_flags =
      shared ? reinterpret_cast<uint8_t*>(static_cast<char*>(workspace) + w.flags_offset)
             : nullptr;
  a->order = w.bytes > 0 && (nwg > kOrderMinWorkgroups || shared)
                 ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + w.order_offset)
                 : nullptr;
  *num_workgroups = nwg;
  return 1;  // ready to launch
}

ReduceKernelArgs reduce_args(const DecodeKernelArgs& a, uint32_t head_dim) {
  ReduceKernelArgs r;
  r.context_lens = a.context_lens;
  r.ws_o = a.ws_o;
  r.ws_ml = a.ws_ml;
  r.out = a.out;
  r.num_seqs = a.num_seqs;
  r.num_q_heads = a.num_q_heads;
  r.head_dim = head_dim;
  r.max_parts = a.max_parts;
  r.part_tokens = a.part_tokens;
  r.max_context_len = a.max_context_len;
  return r;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HPKV_OK : HPKV_ERR_HIP; }

// The partition pass, then the reduce when some sequence spans several partitions.
int launch_decode(int dtype, uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                  hipStream_t s) {
  hipError_t e = hpkv::launch_decode_partitions(dtype, head_dim, a, nwg, s);
  if (e != hipSuccess) return HPKV_ERR_HIP;
  if (a.max_parts > 1) e = hpkv::launch_decode_reduce(dtype, reduce_args(a, head_dim), s);
  return hip_status(e);
}

}  // namespace

extern "C" {

const char* hpkv_status_string(int status) {
  switch (status) {
    case HPKV_OK: return "ok";
    case HPKV_ERR_NULL: return "a required pointer is NULL";
    case HPKV_ERR_INVALID_ARG: return "invalid size or enum argument";
    case HPKV_ERR_INVALID_INDEX: return "index buffer contents break an invariant";
    case HPKV_ERR_UNSUPPORTED: return "unsupported shape";
    case HPKV_ERR_HIP: return "HIP runtime error at launch";
    case HPKV_ERR_WORKSPACE: return "workspace missing or too small";
    case HPKV_ERR_SCRATCH_LIMIT:
      return "batch needs more decode scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int hpkv_validate_index_buffers(int index_type, uint64_t num_pages, uint64_t num_seqs,
                                const void* seq_ptr, const void* block_table,
                                uint64_t block_table_len, const int32_t* context_lens,
                                uint32_t page_size) {
  if (!valid_index(index_type)) return HPKV_ERR_INVALID_ARG;
  if (!seq_ptr || (block_table_len > 0 && !block_table)) return HPKV_ERR_NULL;
  if (context_lens && page_size == 0) return HPKV_ERR_INVALID_ARG;
  if (read_index(index_type, seq_ptr, 0) != 0) return HPKV_ERR_INVALID_INDEX;
  for (uint64_t s = 0; s < num_seqs; ++s)
    if (read_index(index_type, seq_ptr, s + 1) < read_index(index_type, seq_ptr, s))
      return HPKV_ERR_INVALID_INDEX;
  if (read_index(index_type, seq_ptr, num_seqs) != block_table_len) return HPKV_ERR_INVALID_INDEX;
  for (uint64_t k = 0; k < block_table_len; ++k)
    if (read_index(index_type, block_table, k) >= num_pages) return HPKV_ERR_INVALID_INDEX;
  if (context_lens) {
    for (uint64_t s = 0; s < num_seqs; ++s) {
      const uint64_t pages =
          read_index(index_type, seq_ptr, s + 1) - read_index(index_type, seq_ptr, s);
      if (context_lens[s] < 0 || uint64_t(context_lens[s]) > pages * page_size)
        return HPKV_ERR_INVALID_INDEX;
    }
  }
  return HPKV_OK;
}

int hpkv_element_offset(int index_type, uint64_t s, uint64_t t, uint32_t h, uint32_t d,
                        uint32_t page_size, uint64_t num_pages, uint32_t num_heads,
                        uint32_t head_dim, const void* block_table, uint64_t block_table_len,
                        const void* seq_ptr, uint64_t num_seqs, uint64_t* flat_out) {
  if (!valid_index(index_type)) return HPKV_ERR_INVALID_ARG;
  if (!block_table || !seq_ptr || !flat_out) return HPKV_ERR_NULL;
  if (page_size == 0 || num_heads == 0 || head_dim == 0) return HPKV_ERR_INVALID_ARG;
  if (s >= num_seqs || h >= num_heads || d >= head_dim) return HPKV_ERR_INVALID_INDEX;
  const uint64_t first = read_index(index_type, seq_ptr, s);
  const uint64_t last = read_index(index_type, seq_ptr, s + 1);
  const uint64_t page = t / page_size;
  if (last < first || page >= last - first || first + page >= block_table_len)
    return HPKV_ERR_INVALID_INDEX;
  const uint64_t phys = read_index(index_type, block_table, first + page);
  if (phys >= num_pages) return HPKV_ERR_INVALID_INDEX;
  *flat_out = ((phys * page_size + t % page_size) * num_heads + h) * head_dim + d;
  return HPKV_OK;
}

int hpkv_validate_shape(uint32_t rank, const uint64_t* dims) {
  if (rank != 3) return HPKV_ERR_INVALID_ARG;
  if (!dims) return HPKV_ERR_NULL;
  if (dims[1] == 0 || dims[2] == 0) return HPKV_ERR_INVALID_ARG;
  return HPKV_OK;
}

int hpkv_slot_mapping(int index_type, const void* block_table, uint64_t block_table_len,
                      const void* seq_ptr, uint32_t num_seqs, uint32_t page_size,
                      uint64_t num_pages, const int32_t* start_pos, const int64_t* cu_new, uint64_t num_new,
                      int64_t* slots, void* stream) {
  if (!valid_index(index_type)) return HPKV_ERR_INVALID_ARG;
  if (page_size == 0) return HPKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_new == 0) return HPKV_OK;
  if (!seq_ptr || !start_pos || !cu_new || !slots) return HPKV_ERR_NULL;
  if (block_table_len > 0 && !block_table) return HPKV_ERR_NULL;
  if (num_new > (uint64_t(0x7fffffff) * 256)) return HPKV_ERR_UNSUPPORTED;
  return hip_status(hpkv::launch_slot_mapping(
      index_type == HPKV_INDEX_U64, block_table, block_table_len, seq_ptr, num_seqs, page_size,
      num_pages, start_pos, cu_new, num_new, slots, static_cast<hipStream_t>(stream)));
}

int hpkv_store_kvcache(int dtype, const void* key, const void* value, void* k_cache,
                       void* v_cache, const int64_t* slots, uint64_t num_tokens,
                       uint32_t page_size, uint64_t num_pages, uint32_t num_kv_heads,
                       uint32_t head_dim, void* stream) {
  if (!valid_dtype(dtype)) return HPKV_ERR_INVALID_ARG;
  if (page_size == 0 || num_pages == 0 || num_kv_heads == 0 || head_dim == 0)
    return HPKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return HPKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slots) return HPKV_ERR_NULL;
  const uint64_t row_bytes = uint64_t(num_kv_heads) * head_dim * hpkv::dtype_bytes(dtype);
  const uint64_t num_slots = num_pages * page_size;
  if (num_slots > uint64_t(INT64_MAX) / row_bytes) return HPKV_ERR_INVALID_ARG;
  // widest copy unit that divides the row and every base address
  const uintptr_t align = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
                          reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | uintptr_t(row_bytes);
  const int chunk = (align % 16 == 0) ? 16 : (align % 4 == 0) ? 4 : 2;
  return hip_status(hpkv::launch_store(chunk, key, value, k_cache, v_cache, slots, num_tokens,
                                       row_bytes / chunk, int64_t(num_slots),
                                       static_cast<hipStream_t>(stream)));
}

uint32_t hpkv_paged_attention_decode_partition_tokens(int dtype, uint32_t num_seqs,
                                                      uint32_t num_q_heads,
                                                      uint32_t num_kv_heads, uint32_t head_dim,
                                                      uint32_t page_size,
                                                      uint32_t max_context_len) {
  if (!valid_dtype(dtype) || num_q_heads == 0 || num_kv_heads == 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  return plan_decode(dtype, false, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     max_context_len)
      .part_tokens;
}

uint32_t hpkv_paged_attention_decode_quant_partition_tokens(int dtype, int kv_type,
                                                            uint32_t num_seqs,
                                                            uint32_t num_q_heads,
                                                            uint32_t num_kv_heads,
                                                            uint32_t head_dim, uint32_t page_size,
                                                            uint32_t max_context_len) {
  if (!valid_dtype(dtype) || (kv_type != HPKV_KV_I8 && kv_type != HPKV_KV_FP8_E4M3) ||
      num_q_heads == 0 || num_kv_heads == 0 || num_q_heads % num_kv_heads != 0 || page_size == 0)
    return 0;
  return plan_decode(dtype, true, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     max_context_len)
      .part_tokens;
}

size_t hpkv_paged_attention_decode_workspace_size(int dtype, uint32_t num_seqs,
                                                  uint32_t num_q_heads, uint32_t head_dim,
                                                  uint32_t page_size, uint32_t max_context_len) {
  if (!valid_dtype(dtype) || page_size == 0) return 0;
  // sized for the smallest partition, so it covers every shape
  return workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, kPartTokens).bytes;
}

int hpkv_paged_attention_decode_partitions(int dtype, int index_type, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const void* block_table, uint64_t block_table_len,
                                           const void* seq_ptr, const int32_t* context_lens,
                                           uint32_t num_seqs, uint32_t num_q_heads,
                                           uint32_t num_kv_heads, uint32_t head_dim,
                                           uint32_t page_size, uint64_t num_pages, float scale,
                                           uint32_t max_context_len, void* workspace,
                                           size_t workspace_bytes, void* out, void* stream) {
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  const int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table,
                                block_table_len, seq_ptr, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, scale,
                                max_context_len, workspace, workspace_bytes, out, &a, &nwg);
  if (st <= 0) return st;
  return hip_status(
      hpkv::launch_decode_partitions(dtype, head_dim, a, nwg, static_cast<hipStream_t>(stream)));
}

int hpkv_paged_attention_decode_reduce(int dtype, const int32_t* context_lens, uint32_t num_seqs,
                                       uint32_t num_q_heads, uint32_t num_kv_heads,
                                       uint32_t head_dim, uint32_t page_size,
                                       uint32_t max_context_len, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream) {
  if (!valid_dtype(dtype)) return HPKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return HPKV_OK;
  if (!context_lens || !out) return HPKV_ERR_NULL;
  if (num_q_heads == 0 || num_kv_heads == 0 || head_dim == 0 || page_size == 0)
    return HPKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return HPKV_ERR_INVALID_ARG;
  if (max_context_len > 0x7fffffffu) return HPKV_ERR_INVALID_ARG;
  if (!decode_head_dim_supported(dtype, head_dim)) return HPKV_ERR_UNSUPPORTED;
  const uint32_t part_tokens = plan_decode(dtype, false, num_seqs, num_q_heads, num_kv_heads,
                                           head_dim, page_size, max_context_len)
                                   .part_tokens;
  const WorkspaceLayout w =
      workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, part_tokens);
  if (w.bytes == 0) return HPKV_OK;  // single partition: nothing to merge
  if (!workspace || workspace_bytes < w.bytes) return HPKV_ERR_WORKSPACE;
  ReduceKernelArgs r;
  r.context_lens = context_lens;
  r.ws_ml = reinterpret_cast<const float2*>(static_cast<char*>(workspace) + w.ml_offset);
  r.ws_o = reinterpret_cast<const float*>(static_cast<char*>(workspace) + w.o_offset);
  r.out = out;
  r.num_seqs = num_seqs;
  r.num_q_heads = num_q_heads;
  r.head_dim = head_dim;
  r.max_parts = max_parts_for(max_context_len, part_tokens);
  r.part_tokens = part_tokens;
  r.max_context_len = max_context_len;
  return hip_status(hpkv::launch_decode_reduce(dtype, r, static_cast<hipStream_t>(stream)));
}

int hpkv_paged_attention_decode(int dtype, int index_type, const void* q, const void* k_cache,
                                const void* v_cache, const void* block_table,
                                uint64_t block_table_len, const void* seq_ptr,
                                const int32_t* context_lens, uint32_t num_seqs,
                                uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                                uint32_t page_size, uint64_t num_pages, float scale,
                                uint32_t max_context_len, void* workspace, size_t workspace_bytes,
                                void* out, void* stream) {
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  const int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table,
                                block_table_len, seq_ptr, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, scale,
                                max_context_len, workspace, workspace_bytes, out, &a, &nwg);
  if (st <= 0) return st;
  return launch_decode(dtype, head_dim, a, nwg, static_cast<hipStream_t>(stream));
}

int hpkv_paged_attention_decode_shared(int dtype, int index_type, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const void* block_table, uint64_t block_table_len,
                                       const void* seq_ptr, const int32_t* context_lens,
                                       uint32_t num_seqs, uint32_t num_q_heads,
                                       uint32_t num_kv_heads, uint32_t head_dim,
                                       uint32_t page_size, uint64_t num_pages, float scale,
                                       uint32_t max_context_len, void* workspace,
                                       size_t workspace_bytes, void* out, void* stream) {
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  const int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table,
                                block_table_len, seq_ptr, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, scale,
                                max_context_len, workspace, workspace_bytes, out, &a, &nwg, -1,
                                true);
  if (st <= 0) return st;
  return launch_decode(dtype, head_dim, a, nwg, static_cast<hipStream_t>(stream));
}

size_t hpkv_paged_attention_decode_noalloc_max_workspace(void) {
  return hpkv::kNoallocScratchBytes;
}

int hpkv_paged_attention_decode_noalloc(int dtype, int index_type, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const void* block_table, uint64_t block_table_len,
                                        const void* seq_ptr, const int32_t* context_lens,
                                        uint32_t num_seqs, uint32_t num_q_heads,
                                        uint32_t num_kv_heads, uint32_t head_dim,
                                        uint32_t page_size, uint64_t num_pages, float scale,
                                        uint32_t max_context_len, void* out, void* stream) {
  const size_t need = hpkv_paged_attention_decode_workspace_size(
      dtype, num_seqs, num_q_heads, head_dim, page_size, max_context_len);
  if (need > hpkv::kNoallocScratchBytes) return HPKV_ERR_SCRATCH_LIMIT;
  // every argument check first, without a workspace: HPKV_ERR_WORKSPACE then
  // only says that this batch needs one
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table, block_table_len,
                          seq_ptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          page_size, num_pages, scale, max_context_len, nullptr, 0, out, &a,
                          &nwg);
  if (st != 1 && st != HPKV_ERR_WORKSPACE) return st;
  void* scratch = nullptr;
  if (hpkv::noalloc_scratch(&scratch) != hipSuccess) return HPKV_ERR_HIP;
  if (st == HPKV_ERR_WORKSPACE) {
    st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table, block_table_len,
                        seq_ptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        page_size, num_pages, scale, max_context_len, scratch,
                        hpkv::kNoallocScratchBytes, out, &a, &nwg);
    if (st <= 0) return st;
  }
  return launch_decode(dtype, head_dim, a, nwg, static_cast<hipStream_t>(stream));
}

int hpkv_paged_attention_decode_step(int dtype, int index_type, const void* q,
                                     const void* new_key, const void* new_value, void* k_cache,
                                     void* v_cache, const void* block_table,
                                     uint64_t block_table_len, const void* seq_ptr,
                                     const int32_t* context_lens, uint32_t num_seqs,
                                     uint32_t num_q_heads, uint32_t num_kv_heads,
                                     uint32_t head_dim, uint32_t page_size, uint64_t num_pages,
                                     float scale, uint32_t max_context_len, int64_t* slots_out,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream) {
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  const int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table,
                                block_table_len, seq_ptr, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, scale,
                                max_context_len, workspace, workspace_bytes, out, &a, &nwg);
  if (st <= 0) return st;
  if (!new_key || !new_value) return HPKV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(new_key) | reinterpret_cast<uintptr_t>(new_value)) % 16 != 0)
    return HPKV_ERR_INVALID_ARG;
  a.new_k = new_key;
  a.new_v = new_value;
  a.slots_out = slots_out;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hpkv::launch_decode_partitions(dtype, head_dim, a, nwg, s);
  if (e != hipSuccess) return HPKV_ERR_HIP;
  if (a.max_parts > 1) e = hpkv::launch_decode_reduce(dtype, reduce_args(a, head_dim), s);
  return hip_status(e);
}

int hpkv_paged_attention_prefill(int dtype, int index_type, const void* q, const void* k_cache,
                                 const void* v_cache, const void* block_table,
                                 uint64_t block_table_len, const void* seq_ptr,
                                 const int32_t* q_start, const int64_t* cu_q, uint32_t num_seqs,
                                 uint64_t num_q_tokens, uint32_t num_q_heads,
                                 uint32_t num_kv_heads, uint32_t head_dim, uint32_t page_size,
                                 uint64_t num_pages, float scale, uint32_t max_q_len, void* out,
                                 void* stream) {
  if (!valid_dtype(dtype) || !valid_index(index_type)) return HPKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_q_tokens == 0) return HPKV_OK;
  if (!q || !k_cache || !v_cache || !seq_ptr || !q_start || !cu_q || !out) return HPKV_ERR_NULL;
  if (block_table_len > 0 && !block_table) return HPKV_ERR_NULL;
  if (num_q_heads == 0 || num_kv_heads == 0 || head_dim == 0 || page_size == 0 ||
      num_pages == 0 || max_q_len == 0)
    return HPKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return HPKV_ERR_INVALID_ARG;
  if (page_size > 0x7fffffffu || max_q_len > 0x7fffffffu) return HPKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return HPKV_ERR_INVALID_ARG;  // NaN scale
  if (!hpkv::prefill_head_dim_supported(dtype, head_dim)) return HPKV_ERR_UNSUPPORTED;
  // the kernel keeps pool rows (page * page_size + offset) in 32 bits
  if (num_pages > 0xffffffffull / page_size) return HPKV_ERR_UNSUPPORTED;
  const uint32_t group = num_q_heads / num_kv_heads;
  const uint32_t rows = hpkv::prefill_rows_per_workgroup(dtype, head_dim);
  if (group > rows) return HPKV_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) % 16 != 0)
    return HPKV_ERR_INVALID_ARG;

  // no chunk can hold more rows than the call has
  const uint64_t qmax = max_q_len < num_q_tokens ? max_q_len : num_q_tokens;
  const uint32_t block_positions = rows / group;
  const uint64_t pos_blocks = (qmax + block_positions - 1) / block_positions;
  const uint64_t work = pos_blocks * num_kv_heads * num_seqs;
  const uint64_t nwg = (work + 7) / 8 * 8;  // a multiple of the 8 XCDs
  if (nwg > 0x7fffffffull) return HPKV_ERR_UNSUPPORTED;

  hpkv::PrefillKernelArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.block_table = block_table;
  a.seq_ptr = seq_ptr;
  a.q_start = q_start;
  a.cu_q = cu_q;
  a.block_table_len = block_table_len;
  a.num_pages = num_pages;
  a.num_q_tokens = num_q_tokens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.page_size = page_size;
  a.group = group;
  a.block_positions = block_positions;
  a.pos_blocks = uint32_t(pos_blocks);
  a.max_q_len = max_q_len;
  a.num_work = uint32_t(work);
  a.page_div = hpkv::make_fastdiv(page_size);
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a.idx64 = index_type == HPKV_INDEX_U64;
  return hip_status(hpkv::launch_prefill(dtype, head_dim, a, uint32_t(nwg),
                                         static_cast<hipStream_t>(stream)));
}

int hpkv_store_kvcache_quant(int dtype, int kv_type, const void* key, const void* value,
                             void* k_cache, void* v_cache, const float* k_scale,
                             const float* k_zero, const float* v_scale, const float* v_zero,
                             const int64_t* slots, uint64_t num_tokens, uint32_t page_size,
                             uint64_t num_pages, uint32_t num_kv_heads, uint32_t head_dim,
                             void* stream) {
  if (!valid_dtype(dtype)) return HPKV_ERR_INVALID_ARG;
  if (kv_type != HPKV_KV_I8 && kv_type != HPKV_KV_FP8_E4M3) return HPKV_ERR_INVALID_ARG;
  if (page_size == 0 || num_pages == 0 || num_kv_heads == 0 || head_dim == 0)
    return HPKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return HPKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slots || !k_scale || !k_zero || !v_scale ||
      !v_zero)
    return HPKV_ERR_NULL;
  if (head_dim % 8 != 0) return HPKV_ERR_UNSUPPORTED;
  const uint64_t row_elems = uint64_t(num_kv_heads) * head_dim;
  if (num_pages * page_size > uint64_t(INT64_MAX) / row_elems) return HPKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value)) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 8 != 0)
    return HPKV_ERR_INVALID_ARG;
  return hip_status(hpkv::launch_store_quant(dtype, kv_type, key, value, k_cache, v_cache,
                                             k_scale, k_zero, v_scale, v_zero, slots, num_tokens,
                                             page_size, num_pages, num_kv_heads, head_dim,
                                             static_cast<hipStream_t>(stream)));
}

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
                                      size_t workspace_bytes, void* out, void* stream) {
  DecodeKernelArgs a;
  uint64_t nwg = 0;
  const int st = prepare_decode(dtype, index_type, q, k_cache, v_cache, block_table,
                                block_table_len, seq_ptr, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, scale,
                                max_context_len, workspace, workspace_bytes, out, &a, &nwg,
                                kv_type);
  if (st <= 0) return st;
  if (!k_scale || !k_zero || !v_scale || !v_zero) return HPKV_ERR_NULL;
  a.k_scale = k_scale;
  a.k_zero = k_zero;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hpkv::launch_decode_partitions_quant(dtype, kv_type, head_dim, a, nwg, s);
  if (e != hipSuccess) return HPKV_ERR_HIP;
  if (a.max_parts > 1) e = hpkv::launch_decode_reduce(dtype, reduce_args(a, head_dim), s);
  return hip_status(e);
}

int hpkv_read_ceiling(const void* buf, uint64_t bytes, uint32_t row_bytes,
                      uint64_t stride_bytes, uint32_t rows_per_workgroup, uint32_t* sink,
                      void* stream) {
  if (!buf || !sink) return HPKV_ERR_NULL;
  if (row_bytes < 16 || row_bytes > 4096 || (row_bytes & (row_bytes - 1)) != 0)
    return HPKV_ERR_INVALID_ARG;
  if (stride_bytes < row_bytes || stride_bytes % row_bytes != 0) return HPKV_ERR_INVALID_ARG;
  if (rows_per_workgroup == 0) return HPKV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return HPKV_ERR_INVALID_ARG;
  return hip_status(hpkv::launch_read_ceiling(buf, bytes, row_bytes, stride_bytes,
                                              rows_per_workgroup, sink,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
