// hpkv CPU oracle: a plain, slow, deliberately unoptimised statement of what the
// block-paged KV cache hot path computes. This is TEST INFRASTRUCTURE: only the
// tests, the smoke check and the CPU-baseline leg of the benchmark may load it.
// It shares no code, header, table or constant with the HIP library; the two
// are compared against each other, never built from each other.
//
// Sources (web pages, cited by title and section):
//   [HUR]  "Block-Paged KV Cache" (Hurray format documentation, cookbook):
//          sections "The three buffers", "Element lookup through the block
//          table", "Validating the storage invariants".
//   [INT]  "Paged KV Cache · AI infra interview lesson": sections "Walk the
//          Shapes First", "Step 1: slot_mapping and store_kvcache",
//          "Step 2: paged_attention_decode", "Common Pitfalls".
//   [LLM]  "LLM Inference Engineering & Economics", Chapter 2 (KV cache,
//          memory hierarchy, continuous batching, and PagedAttention):
//          sections "What the KV cache actually stores", "Sliding windows,
//          GQA, and hybrid caches change the equation".
//
// Floating point: every score, softmax weight and output is computed in double
// from inputs widened exactly from their storage type; the result is rounded
// once, to nearest-even, to the storage type of q.
//
// Readings taken where the pages leave a step open (each also listed in the
// design notes):
//   * The block table is the CSR pair (block_table, seq_ptr) of [HUR].
//   * Positions whose logical page is not in the sequence's slice give slot -1.
//   * Only the first ceil(ctx/page_size) pages of a slice are read ([INT] Step 2
//     slices the table before indexing); extra pages are ignored.
//   * ctx_len == 0 gives an all-zero output row (the empty sum of [INT] Step 2).
//   * A store skips slot -1 and any slot outside [0, num_pages*page_size);
//     repeated slots resolve last-writer-wins in token order.
//   * GQA: query head h reads KV head h / (Hq/Hkv) ([INT] Step 2).
//   * scale multiplies the q.k dot product ([INT] Step 2).
//   * Quantized pools ([HUR] "Quantization compatibility": per-block-affine
//     along the paged axis with block_size == page_size, so every physical
//     page slot carries its own scales): elements are int8 or OCP fp8 E4M3
//     ("e4m3fn"); each page holds, per KV head, an fp32 scale and zero point
//     for K and for V, and an element with code q stands for
//     scale * (value(q) - zero). The store quantizes t = x / scale + zero
//     (both steps in fp32) to the nearest code, ties to even, saturating at
//     the type's range (int8: [-128, 127]; e4m3fn: +-448).
//   * Chunked prefill: the query at position p of a chunk attends to tokens
//     0..p of its own sequence (causal softmax attention), all read from the
//     pool, so the chunk's own K/V rows are stored before attention ([INT]
//     Step 1 chunked prefill / prefix hit, then the gather of Step 2).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// Status codes of this oracle (independent of the library's own codes).
enum : int {
  ORC_OK = 0,
  ORC_BAD_ARG = 1,
  ORC_SEQ_PTR_FIRST = 2,      // seq_ptr[0] != 0
  ORC_SEQ_PTR_ORDER = 3,      // seq_ptr decreases somewhere
  ORC_SEQ_PTR_LAST = 4,       // seq_ptr[num_seqs] != block_table length
  ORC_PAGE_RANGE = 5,         // some block_table entry >= num_pages
  ORC_CTX_RANGE = 6,          // a context length is negative or exceeds its slice
  ORC_OUT_OF_RANGE = 7,       // an element lookup coordinate is out of range
};

// Element storage types understood by the oracle (the last two only for the
// K/V pools).
enum : int { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_I8 = 3, ORC_FP8 = 4 };

uint64_t read_index(int index_bytes, const void* p, uint64_t i) {
  if (index_bytes == 4) return static_cast<const uint32_t*>(p)[i];
  return static_cast<const uint64_t*>(p)[i];
}

// ---- exact widening of stored elements to double -------------------------

double widen_f32(uint32_t bits) {
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

// bfloat16 is the upper half of an IEEE binary32.
double widen_bf16(uint16_t bits) { return widen_f32(uint32_t(bits) << 16); }

// IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double widen_f16(uint16_t bits) {
  const int sign = bits >> 15;
  const int expo = (bits >> 10) & 0x1f;
  const int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = std::ldexp(double(frac), -24);  // subnormal: frac * 2^-24
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = std::ldexp(double(1024 + frac), expo - 25);
  }
  return sign ? -mag : mag;
}

double load_elem(int dtype, const void* base, uint64_t idx) {
  if (dtype == ORC_F32) return widen_f32(static_cast<const uint32_t*>(base)[idx]);
  const uint16_t b = static_cast<const uint16_t*>(base)[idx];
  return dtype == ORC_BF16 ? widen_bf16(b) : widen_f16(b);
}

// OCP 8-bit float E4M3 in its "fn" variant: 1 sign bit, 4 exponent bits with
// bias 7, 3 fraction bits. Exponent 0 holds subnormals (frac/8 * 2^-6); the
// pattern with every exponent and fraction bit set is NaN; there is no
// infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
double widen_fp8_e4m3(uint8_t bits) {
  const int sign = bits >> 7;
  const int expo = (bits >> 3) & 0xf;
  const int frac = bits & 0x7;
  double mag;
  if (expo == 0xf && frac == 0x7) {
    mag = NAN;
  } else if (expo == 0) {
    mag = std::ldexp(double(frac), -9);  // frac/8 * 2^-6
  } else {
    mag = std::ldexp(double(8 + frac), expo - 10);  // (1 + frac/8) * 2^(expo-7)
  }
  return sign ? -mag : mag;
}

// The value a quantized code stands for before the affine map.
double code_value(int kv_type, uint8_t code) {
  return kv_type == ORC_I8 ? double(int8_t(code)) : widen_fp8_e4m3(code);
}

// Quantizes fp32 t to a code of kv_type: the nearest representable value,
// ties to even, saturating at the largest finite magnitude; NaN gives the NaN
// code for fp8 and 0 for int8. For fp8 the search runs over every finite
// code, so no rounding shortcut is involved.
uint8_t quantize_code(int kv_type, float t) {
  if (kv_type == ORC_I8) {
    if (std::isnan(t)) return 0;
    double r = std::nearbyint(double(t));  // default rounding mode: ties to even
    if (r < -128.0) r = -128.0;
    if (r > 127.0) r = 127.0;
    return uint8_t(int8_t(int(r)));
  }
  if (std::isnan(t)) return 0x7f;
  const double a = std::fabs(double(t));
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7e; ++c) {  // every finite non-negative code, in increasing value
    const double err = std::fabs(widen_fp8_e4m3(uint8_t(c)) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  if (a >= 448.0) best = 0x7e;  // saturate
  return uint8_t(best | (std::signbit(t) ? 0x80 : 0));
}

// ---- rounding double -> storage type, to nearest, ties to even -------------
// A binary floating-point format with `p` significand bits (implicit bit
// included), smallest normal exponent `emin` and largest exponent `emax`.
// Values are snapped to the quantum of their binade (the subnormal quantum
// below 2^emin) with rint, which rounds ties to even in the default mode.
double round_to_format(double x, int p, int emin, int emax) {
  if (!std::isfinite(x) || x == 0.0) return x;
  int e;
  std::frexp(x, &e);  // |x| in [2^(e-1), 2^e)
  int lead = e - 1;
  if (lead < emin) lead = emin;
  const double quantum = std::ldexp(1.0, lead - (p - 1));
  const double r = std::rint(x / quantum) * quantum;
  const double max_finite = std::ldexp(2.0 - std::ldexp(1.0, -(p - 1)), emax);
  if (std::fabs(r) > max_finite) return std::copysign(INFINITY, x);
  return r;
}

uint32_t encode_f32(double x) {
  const float f = static_cast<float>(round_to_format(x, 24, -126, 127));
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (std::isnan(x)) u = 0x7fc00000u;
  return u;
}

uint16_t encode_bf16(double x) {
  if (std::isnan(x)) return 0x7fc0;
  const float f = static_cast<float>(round_to_format(x, 8, -126, 127));  // exact
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}

uint16_t encode_f16(double x) {
  if (std::isnan(x)) return 0x7e00;
  const double r = round_to_format(x, 11, -14, 15);
  const uint16_t sign = std::signbit(r) ? 0x8000 : 0;
  const double a = std::fabs(r);
  if (std::isinf(a)) return sign | 0x7c00;
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);
  const int lead = e - 1;
  if (lead < -14) {  // subnormal: a = frac * 2^-24
    return sign | static_cast<uint16_t>(std::ldexp(a, 24));
  }
  const uint16_t frac = static_cast<uint16_t>(std::ldexp(a, 10 - lead) - 1024.0);
  return sign | static_cast<uint16_t>((lead + 15) << 10) | frac;
}

void store_elem(int dtype, void* base, uint64_t idx, double x) {
  if (dtype == ORC_F32) {
    static_cast<uint32_t*>(base)[idx] = encode_f32(x);
  } else if (dtype == ORC_BF16) {
    static_cast<uint16_t*>(base)[idx] = encode_bf16(x);
  } else {
    static_cast<uint16_t*>(base)[idx] = encode_f16(x);
  }
}

// Flat page-pool offset of (sequence s, token t, head h, dim e): [HUR] "Element
// lookup through the block table". The pool is
// [num_pages, page_size, num_heads, head_dim] row-major; the token's logical
// page t/page_size is looked up in the sequence's slice of block_table.
// Returns ORC_OK and writes *flat, or an error code.
int element_offset(int index_bytes, uint64_t s, uint64_t t, uint64_t h, uint64_t e,
                   uint64_t page_size, uint64_t num_pages, uint64_t num_heads,
                   uint64_t head_dim, const void* block_table, uint64_t block_table_len,
                   const void* seq_ptr, uint64_t num_seqs, uint64_t* flat) {
  if (page_size == 0 || num_heads == 0 || head_dim == 0) return ORC_BAD_ARG;
  if (s >= num_seqs || h >= num_heads || e >= head_dim) return ORC_OUT_OF_RANGE;
  const uint64_t first = read_index(index_bytes, seq_ptr, s);
  const uint64_t last = read_index(index_bytes, seq_ptr, s + 1);
  const uint64_t page_in_seq = t / page_size;
  const uint64_t offset_in_page = t % page_size;
  if (last < first || page_in_seq >= last - first) return ORC_OUT_OF_RANGE;
  if (first + page_in_seq >= block_table_len) return ORC_OUT_OF_RANGE;
  const uint64_t phys = read_index(index_bytes, block_table, first + page_in_seq);
  if (phys >= num_pages) return ORC_OUT_OF_RANGE;
  *flat = ((phys * page_size + offset_in_page) * num_heads + h) * head_dim + e;
  return ORC_OK;
}

// Row (pool slot) of token t of sequence s: the element offset of (s, t, 0, 0)
// divided by the row width, i.e. block_table[seq_ptr[s] + t/bs]*bs + t%bs.
int token_row(int index_bytes, uint64_t s, uint64_t t, uint64_t page_size, uint64_t num_pages,
              uint64_t num_heads, uint64_t head_dim, const void* block_table,
              uint64_t block_table_len, const void* seq_ptr, uint64_t num_seqs, uint64_t* row) {
  uint64_t flat = 0;
  const int st = element_offset(index_bytes, s, t, 0, 0, page_size, num_pages, num_heads, head_dim,
                                block_table, block_table_len, seq_ptr, num_seqs, &flat);
  if (st != ORC_OK) return st;
  *row = flat / (num_heads * head_dim);
  return ORC_OK;
}

struct DecodeArgs {
  int dtype;
  int index_bytes;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* block_table;
  uint64_t block_table_len;
  const void* seq_ptr;
  const int32_t* context_lens;
  uint64_t num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, num_pages;
  double scale;
  void* out;        // [B, Hq, d] in dtype
  double* out_f64;  // [B, Hq, d] unrounded, may be null
  // Pool element type (ORC_F32/F16/BF16: the same as dtype; ORC_I8/ORC_FP8:
  // quantized, with per (page, KV head) scales and zero points for K and V).
  int kv_type;
  const float* k_scale;
  const float* k_zero;
  const float* v_scale;
  const float* v_zero;
};

// Element e of KV head g in pool row `row` (= page * page_size + offset), as the
// real number it stands for.
double kv_elem(const DecodeArgs& a, const void* pool, const float* sc, const float* zr,
               uint64_t row, uint64_t g, uint64_t e) {
  const uint64_t idx = (row * a.num_kv_heads + g) * a.head_dim + e;
  if (a.kv_type != ORC_I8 && a.kv_type != ORC_FP8) return load_elem(a.dtype, pool, idx);
  const uint64_t p = (row / a.page_size) * a.num_kv_heads + g;
  const double v = code_value(a.kv_type, static_cast<const uint8_t*>(pool)[idx]);
  return double(sc[p]) * (v - double(zr[p]));
}

// One sequence of [INT] "Step 2: paged_attention_decode": gather the first
// ctx tokens of K and V through the block table, then for every query head
// take softmax(scale * q.K^T) and weight V with it. Two passes (max, then
// weighted sums), all in double.
int decode_one_sequence(const DecodeArgs& a, uint64_t s) {
  const uint64_t Hq = a.num_q_heads, Hkv = a.num_kv_heads, d = a.head_dim;
  const uint64_t group = Hq / Hkv;
  const int32_t n_signed = a.context_lens[s];
  const uint64_t first = read_index(a.index_bytes, a.seq_ptr, s);
  const uint64_t last = read_index(a.index_bytes, a.seq_ptr, s + 1);
  if (n_signed < 0 || last < first) return ORC_CTX_RANGE;
  const uint64_t n = static_cast<uint64_t>(n_signed);
  if (n > (last - first) * a.page_size) return ORC_CTX_RANGE;

  std::vector<uint64_t> rows(n);
  for (uint64_t t = 0; t < n; ++t) {
    const int st = token_row(a.index_bytes, s, t, a.page_size, a.num_pages, Hkv, d, a.block_table,
                             a.block_table_len, a.seq_ptr, a.num_seqs, &rows[t]);
    if (st != ORC_OK) return st;
  }
  std::vector<double> z(n), o(d);
  for (uint64_t h = 0; h < Hq; ++h) {
    const uint64_t g = h / group;  // consecutive GQA grouping
    const uint64_t q_base = (s * Hq + h) * d;
    double zmax = -INFINITY;
    for (uint64_t t = 0; t < n; ++t) {
      double dot = 0.0;
      for (uint64_t e = 0; e < d; ++e)
        dot += load_elem(a.dtype, a.q, q_base + e) *
               kv_elem(a, a.k_cache, a.k_scale, a.k_zero, rows[t], g, e);
      z[t] = dot * a.scale;
      zmax = std::max(zmax, z[t]);
    }
    double denom = 0.0;
    std::fill(o.begin(), o.end(), 0.0);
    for (uint64_t t = 0; t < n; ++t) {
      const double w = std::exp(z[t] - zmax);
      denom += w;
      for (uint64_t e = 0; e < d; ++e)
        o[e] += w * kv_elem(a, a.v_cache, a.v_scale, a.v_zero, rows[t], g, e);
    }
    for (uint64_t e = 0; e < d; ++e) {
      const double val = n == 0 ? 0.0 : o[e] / denom;
      if (a.out) store_elem(a.dtype, a.out, q_base + e, val);
      if (a.out_f64) a.out_f64[q_base + e] = val;
    }
  }
  return ORC_OK;
}

int run_decode(const DecodeArgs& a, int num_threads);

}  // namespace

extern "C" {

// [HUR] "Validating the storage invariants": seq_ptr[0] == 0, seq_ptr never
// decreases, seq_ptr[num_seqs] equals the block_table length, and every page id
// is below num_pages. An empty batch (num_seqs == 0, seq_ptr == [0]) passes.
// When context_lens is given, each length must also be non-negative and fit in
// its slice (ctx <= pages_in_slice * page_size).
int orc_validate_index_buffers(int index_bytes, uint64_t num_pages, uint64_t num_seqs,
                               const void* seq_ptr, const void* block_table,
                               uint64_t block_table_len, const int32_t* context_lens,
                               uint64_t page_size) {
  if ((index_bytes != 4 && index_bytes != 8) || seq_ptr == nullptr) return ORC_BAD_ARG;
  if (block_table_len > 0 && block_table == nullptr) return ORC_BAD_ARG;
  if (read_index(index_bytes, seq_ptr, 0) != 0) return ORC_SEQ_PTR_FIRST;
  for (uint64_t s = 0; s < num_seqs; ++s)
    if (read_index(index_bytes, seq_ptr, s + 1) < read_index(index_bytes, seq_ptr, s))
      return ORC_SEQ_PTR_ORDER;
  if (read_index(index_bytes, seq_ptr, num_seqs) != block_table_len) return ORC_SEQ_PTR_LAST;
  for (uint64_t k = 0; k < block_table_len; ++k)
    if (read_index(index_bytes, block_table, k) >= num_pages) return ORC_PAGE_RANGE;
  if (context_lens != nullptr) {
    for (uint64_t s = 0; s < num_seqs; ++s) {
      const uint64_t pages =
          read_index(index_bytes, seq_ptr, s + 1) - read_index(index_bytes, seq_ptr, s);
      if (context_lens[s] < 0 || uint64_t(context_lens[s]) > pages * page_size)
        return ORC_CTX_RANGE;
    }
  }
  return ORC_OK;
}

// [HUR] "Element lookup through the block table".
int orc_element_offset(int index_bytes, uint64_t s, uint64_t t, uint64_t h, uint64_t e,
                       uint64_t page_size, uint64_t num_pages, uint64_t num_heads,
                       uint64_t head_dim, const void* block_table, uint64_t block_table_len,
                       const void* seq_ptr, uint64_t num_seqs, uint64_t* flat) {
  if (block_table == nullptr || seq_ptr == nullptr || flat == nullptr) return ORC_BAD_ARG;
  if (index_bytes != 4 && index_bytes != 8) return ORC_BAD_ARG;
  return element_offset(index_bytes, s, t, h, e, page_size, num_pages, num_heads, head_dim,
                        block_table, block_table_len, seq_ptr, num_seqs, flat);
}

// [INT] "Walk the Shapes First" / "Step 1" per-token rule over the CSR table:
// new-token row i of sequence s (cu_new[s] <= i < cu_new[s+1]) sits at position
// p = start_pos[s] + (i - cu_new[s]), and its slot is
// block_table[seq_ptr[s] + p/bs]*bs + p%bs. A position whose page is not in the
// sequence's slice, or whose page id is not below num_pages, gets -1 (reading:
// no slot; [HUR] "Validating index buffers" requires every id < num_pages).
int orc_slot_mapping(int index_bytes, const void* block_table, uint64_t block_table_len,
                     const void* seq_ptr, uint64_t num_seqs, uint64_t page_size,
                     uint64_t num_pages, const int32_t* start_pos, const int64_t* cu_new, int64_t* slots) {
  if (page_size == 0 || seq_ptr == nullptr || start_pos == nullptr || cu_new == nullptr)
    return ORC_BAD_ARG;
  for (uint64_t s = 0; s < num_seqs; ++s) {
    const uint64_t first = read_index(index_bytes, seq_ptr, s);
    const uint64_t last = read_index(index_bytes, seq_ptr, s + 1);
    for (int64_t i = cu_new[s]; i < cu_new[s + 1]; ++i) {
      const int64_t p = int64_t(start_pos[s]) + (i - cu_new[s]);
      int64_t slot = -1;
      if (p >= 0 && last >= first) {
        const uint64_t page_in_seq = uint64_t(p) / page_size;
        if (page_in_seq < last - first && first + page_in_seq < block_table_len) {
          const uint64_t phys = read_index(index_bytes, block_table, first + page_in_seq);
          if (phys < num_pages) slot = int64_t(phys * page_size + uint64_t(p) % page_size);
        }
      }
      slots[i] = slot;
    }
  }
  return ORC_OK;
}

// [INT] "Step 1": store_kvcache. The caches are viewed as
// [num_pages*page_size, num_heads*head_dim]; every new-token row whose slot is
// not -1 is copied bit for bit into that slot, for K and for V. Token order,
// last writer wins. Slots outside the pool are skipped and counted.
int64_t orc_store_kvcache(uint64_t elem_size, const void* key, const void* value, void* k_cache,
                          void* v_cache, const int64_t* slots, uint64_t num_tokens,
                          uint64_t page_size, uint64_t num_pages, uint64_t num_heads,
                          uint64_t head_dim) {
  const uint64_t row_bytes = num_heads * head_dim * elem_size;
  const int64_t num_slots = int64_t(num_pages * page_size);
  int64_t skipped_invalid = 0;
  for (uint64_t i = 0; i < num_tokens; ++i) {
    const int64_t slot = slots[i];
    if (slot == -1) continue;
    if (slot < 0 || slot >= num_slots) {
      ++skipped_invalid;
      continue;
    }
    std::memcpy(static_cast<char*>(k_cache) + uint64_t(slot) * row_bytes,
                static_cast<const char*>(key) + i * row_bytes, row_bytes);
    std::memcpy(static_cast<char*>(v_cache) + uint64_t(slot) * row_bytes,
                static_cast<const char*>(value) + i * row_bytes, row_bytes);
  }
  return skipped_invalid;
}

// [INT] "Step 2": paged_attention_decode for a batch, one query per sequence.
// q and out are [B, Hq, d]; the caches are [num_pages, page_size, Hkv, d].
// `out` (storage dtype, nullable) receives the rounded result and `out_f64`
// (nullable) the unrounded double result. Sequences are spread round-robin over
// `num_threads` host threads (a timing convenience; each sequence is computed
// by the same single-threaded routine). Returns ORC_OK or the first error.
int orc_paged_attention_decode(int dtype, int index_bytes, const void* q, const void* k_cache,
                               const void* v_cache, const void* block_table,
                               uint64_t block_table_len, const void* seq_ptr,
                               const int32_t* context_lens, uint64_t num_seqs,
                               uint64_t num_q_heads, uint64_t num_kv_heads, uint64_t head_dim,
                               uint64_t page_size, uint64_t num_pages, double scale, void* out,
                               double* out_f64, int num_threads) {
  if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
  if (index_bytes != 4 && index_bytes != 8) return ORC_BAD_ARG;
  if (num_kv_heads == 0 || head_dim == 0 || page_size == 0) return ORC_BAD_ARG;
  if (num_q_heads % num_kv_heads != 0) return ORC_BAD_ARG;
  DecodeArgs a{dtype,       index_bytes,  q,           k_cache,      v_cache,
               block_table, block_table_len, seq_ptr, context_lens, num_seqs,
               num_q_heads, num_kv_heads, head_dim,    page_size,    num_pages,
               scale,       out,          out_f64,     dtype,        nullptr,
               nullptr,     nullptr,      nullptr};
  return run_decode(a, num_threads);
}

// Decode over quantized pools (kv_type ORC_I8 or ORC_FP8, 1 byte per element,
// [num_pages, page_size, Hkv, d]); scales and zero points are fp32
// [num_pages, Hkv]. Every K/V element is taken at its exact real value
// scale * (value(code) - zero) in double; the rest is the decode above.
int orc_paged_attention_decode_quant(int dtype, int kv_type, int index_bytes, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* k_zero,
                                     const float* v_scale, const float* v_zero,
                                     const void* block_table, uint64_t block_table_len,
                                     const void* seq_ptr, const int32_t* context_lens,
                                     uint64_t num_seqs, uint64_t num_q_heads,
                                     uint64_t num_kv_heads, uint64_t head_dim, uint64_t page_size,
                                     uint64_t num_pages, double scale, void* out, double* out_f64,
                                     int num_threads) {
  if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
  if (kv_type != ORC_I8 && kv_type != ORC_FP8) return ORC_BAD_ARG;
  if (index_bytes != 4 && index_bytes != 8) return ORC_BAD_ARG;
  if (num_kv_heads == 0 || head_dim == 0 || page_size == 0) return ORC_BAD_ARG;
  if (num_q_heads % num_kv_heads != 0) return ORC_BAD_ARG;
  if (!k_scale || !k_zero || !v_scale || !v_zero) return ORC_BAD_ARG;
  DecodeArgs a{dtype,       index_bytes,  q,           k_cache,      v_cache,
               block_table, block_table_len, seq_ptr, context_lens, num_seqs,
               num_q_heads, num_kv_heads, head_dim,    page_size,    num_pages,
               scale,       out,          out_f64,     kv_type,      k_scale,
               k_zero,      v_scale,      v_zero};
  return run_decode(a, num_threads);
}

// Quantized store: every new row with a slot in [0, num_pages*page_size) is
// quantized element by element with the scale and zero point of its page and
// KV head (t = x / scale + zero in fp32, then quantize_code) and written to
// that pool row; rows with any other slot are skipped (last writer wins for
// repeated slots). key/value are [n, Hkv, d] of dtype. Returns the number of
// skipped rows, or -1 on a bad argument.
int64_t orc_store_kvcache_quant(int dtype, int kv_type, const void* key, const void* value,
                                void* k_cache, void* v_cache, const float* k_scale,
                                const float* k_zero, const float* v_scale, const float* v_zero,
                                const int64_t* slots, uint64_t n, uint64_t page_size,
                                uint64_t num_pages, uint64_t num_kv_heads, uint64_t head_dim) {
  if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return -1;
  if (kv_type != ORC_I8 && kv_type != ORC_FP8) return -1;
  if (page_size == 0 || num_kv_heads == 0 || head_dim == 0) return -1;
  const uint64_t num_slots = num_pages * page_size;
  int64_t skipped = 0;
  for (uint64_t i = 0; i < n; ++i) {
    if (slots[i] < 0 || uint64_t(slots[i]) >= num_slots) {
      ++skipped;
      continue;
    }
    const uint64_t slot = uint64_t(slots[i]);
    const uint64_t page = slot / page_size;
    for (uint64_t g = 0; g < num_kv_heads; ++g) {
      const uint64_t p = page * num_kv_heads + g;
      for (uint64_t e = 0; e < head_dim; ++e) {
        const uint64_t src = (i * num_kv_heads + g) * head_dim + e;
        const uint64_t dst = (slot * num_kv_heads + g) * head_dim + e;
        const float xk = float(load_elem(dtype, key, src));
        const float xv = float(load_elem(dtype, value, src));
        const float tk = xk / k_scale[p] + k_zero[p];
        const float tv = xv / v_scale[p] + v_zero[p];
        static_cast<uint8_t*>(k_cache)[dst] = quantize_code(kv_type, tk);
        static_cast<uint8_t*>(v_cache)[dst] = quantize_code(kv_type, tv);
      }
    }
  }
  return skipped;
}

// Exposes the fp8 decoding and the quantizer for the pins.
void orc_fp8_e4m3_decode(const uint8_t* codes, uint64_t n, double* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = widen_fp8_e4m3(codes[i]);
}

void orc_quantize(int kv_type, const float* t, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = quantize_code(kv_type, t[i]);
}

}  // extern "C"

namespace {

int run_decode(const DecodeArgs& a, int num_threads) {
  const uint64_t num_seqs = a.num_seqs;
  if (num_threads < 1) num_threads = 1;
  std::vector<int> status(num_threads, ORC_OK);
  auto work = [&](int k) {
    for (uint64_t s = uint64_t(k); s < num_seqs; s += uint64_t(num_threads)) {
      const int st = decode_one_sequence(a, s);
      if (st != ORC_OK && status[k] == ORC_OK) status[k] = st;
    }
  };
  if (num_threads == 1) {
    work(0);
  } else {
    std::vector<std::thread> pool;
    for (int k = 0; k < num_threads; ++k) pool.emplace_back(work, k);
    for (auto& th : pool) th.join();
  }
  for (int st : status)
    if (st != ORC_OK) return st;
  return ORC_OK;
}

}  // namespace

extern "C" {

// Textbook softmax attention for one query over K/V held contiguously
// ([L, Hkv, d], token-major, never read through a page pool): the dense
// reference that [INT] "Step 2" checks the paged gather against. Query head h
// reads KV head h / (Hq/Hkv). q is [Hq, d]; out is [Hq, d] in double.
int orc_dense_attention(int dtype, const void* q, const void* K, const void* V, uint64_t L,
                        uint64_t num_q_heads, uint64_t num_kv_heads, uint64_t head_dim,
                        double scale, double* out) {
  if (num_kv_heads == 0 || num_q_heads % num_kv_heads != 0) return ORC_BAD_ARG;
  const uint64_t group = num_q_heads / num_kv_heads;
  std::vector<double> logits(L), weights(L);
  for (uint64_t h = 0; h < num_q_heads; ++h) {
    const uint64_t g = h / group;
    for (uint64_t t = 0; t < L; ++t) {
      double acc = 0.0;
      for (uint64_t e = 0; e < head_dim; ++e)
        acc += load_elem(dtype, q, h * head_dim + e) *
               load_elem(dtype, K, (t * num_kv_heads + g) * head_dim + e);
      logits[t] = acc * scale;
    }
    double m = -INFINITY;
    for (uint64_t t = 0; t < L; ++t) m = std::max(m, logits[t]);
    double total = 0.0;
    for (uint64_t t = 0; t < L; ++t) {
      weights[t] = std::exp(logits[t] - m);
      total += weights[t];
    }
    for (uint64_t e = 0; e < head_dim; ++e) {
      double acc = 0.0;
      for (uint64_t t = 0; t < L; ++t)
        acc += weights[t] * load_elem(dtype, V, (t * num_kv_heads + g) * head_dim + e);
      out[h * head_dim + e] = L == 0 ? 0.0 : acc / total;
    }
  }
  return ORC_OK;
}

// Chunked prefill over the paged cache. [INT] "Step 1" describes a prefill
// chunk that may start part-way into a page (a prefix hit, or the second half
// of a chunked prefill); its queries attend causally: the query at position p
// of sequence s sees that sequence's tokens 0..p, read through the block
// table ([INT] "Step 2" gather, [LLM] "What the KV cache actually stores").
// Query rows of sequence s are cu_q[s] .. cu_q[s+1]-1 at positions
// q_start[s] + (i - cu_q[s]). q and out are [Nq, Hq, d]. Each query row is the
// single-query attention of "Step 2" over its first p+1 tokens, computed in
// double and rounded once. Returns ORC_CTX_RANGE if a position is negative or
// beyond the sequence's slice.
int orc_paged_attention_prefill(int dtype, int index_bytes, const void* q, const void* k_cache,
                                const void* v_cache, const void* block_table,
                                uint64_t block_table_len, const void* seq_ptr,
                                const int32_t* q_start, const int64_t* cu_q, uint64_t num_seqs,
                                uint64_t num_q_heads, uint64_t num_kv_heads, uint64_t head_dim,
                                uint64_t page_size, uint64_t num_pages, double scale, void* out,
                                double* out_f64) {
  if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
  if (index_bytes != 4 && index_bytes != 8) return ORC_BAD_ARG;
  if (num_kv_heads == 0 || head_dim == 0 || page_size == 0) return ORC_BAD_ARG;
  if (num_q_heads % num_kv_heads != 0) return ORC_BAD_ARG;
  const uint64_t Hq = num_q_heads, Hkv = num_kv_heads, d = head_dim, group = Hq / Hkv;
  std::vector<double> z, o(d);
  for (uint64_t s = 0; s < num_seqs; ++s) {
    const uint64_t first = read_index(index_bytes, seq_ptr, s);
    const uint64_t last = read_index(index_bytes, seq_ptr, s + 1);
    for (int64_t i = cu_q[s]; i < cu_q[s + 1]; ++i) {
      const int64_t p = int64_t(q_start[s]) + (i - cu_q[s]);
      if (p < 0 || last < first || uint64_t(p) + 1 > (last - first) * page_size) return ORC_CTX_RANGE;
      const uint64_t n = uint64_t(p) + 1;
      std::vector<uint64_t> rows(n);
      for (uint64_t t = 0; t < n; ++t) {
        const int st = token_row(index_bytes, s, t, page_size, num_pages, Hkv, d, block_table,
                                 block_table_len, seq_ptr, num_seqs, &rows[t]);
        if (st != ORC_OK) return st;
      }
      z.assign(n, 0.0);
      for (uint64_t h = 0; h < Hq; ++h) {
        const uint64_t g = h / group;
        const uint64_t q_base = (uint64_t(i) * Hq + h) * d;
        double zmax = -INFINITY;
        for (uint64_t t = 0; t < n; ++t) {
          double dot = 0.0;
          for (uint64_t e = 0; e < d; ++e)
            dot += load_elem(dtype, q, q_base + e) *
                   load_elem(dtype, k_cache, (rows[t] * Hkv + g) * d + e);
          z[t] = dot * scale;
          zmax = std::max(zmax, z[t]);
        }
        double denom = 0.0;
        std::fill(o.begin(), o.end(), 0.0);
        for (uint64_t t = 0; t < n; ++t) {
          const double wgt = std::exp(z[t] - zmax);
          denom += wgt;
          for (uint64_t e = 0; e < d; ++e)
            o[e] += wgt * load_elem(dtype, v_cache, (rows[t] * Hkv + g) * d + e);
        }
        for (uint64_t e = 0; e < d; ++e) {
          if (out) store_elem(dtype, out, q_base + e, o[e] / denom);
          if (out_f64) out_f64[q_base + e] = o[e] / denom;
        }
      }
    }
  }
  return ORC_OK;
}

// Rounds doubles to a storage type (exposed so tests can pin the rounding on
// its own: ties-to-even, subnormals, overflow to infinity).
void orc_round_to_dtype(int dtype, const double* x, uint64_t n, void* out) {
  for (uint64_t i = 0; i < n; ++i) store_elem(dtype, out, i, x[i]);
}

// Widens stored elements to double (pinned the same way).
void orc_widen_dtype(int dtype, const void* x, uint64_t n, double* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = load_elem(dtype, x, i);
}

}  // extern "C"
