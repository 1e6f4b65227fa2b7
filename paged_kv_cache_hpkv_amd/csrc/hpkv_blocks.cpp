// Host block manager: the owner of the physical pages behind block_table.
//
// "Paged KV Cache · AI infra interview lesson", sections "Walk the Shapes
// First" (a sequence needs a new page exactly at the step where its length
// becomes len % page_size == 1) and "Step 5: BlockManager: ref counts and
// chained-hash prefix caching" (pages carry a reference count and, once full,
// a hash chained over the whole prefix, so a later request with the same
// prefix reuses them; a page returns to the free pool only after its last
// reference is released). "LLM Inference Engineering & Economics", Chapter 2,
// sections "PagedAttention separates logical space from physical space",
// "Prefix reuse is another optimization" and "Deterministic evals for this
// layer" (free + allocated = pool; allocated >= pages referenced by live
// tables; no two writable logical pages alias).
//
// Policy (the pages leave these open):
//  * A page is shareable only when full and hashed; a sequence's last,
//    partially filled page is always its own, so every writable page has one
//    owner.
//  * Hash of the i-th full page of a sequence: XXH64 of its page_size token ids
//    (int32, little-endian), seeded with the hash of page i-1 (seed 0 for the
//    first page). A hit also compares the stored token ids, so a hash collision
//    never shares a page.
//  * Free pages are handed out first-freed, first-reused. A freed page keeps
//    its hash registration until it is handed out for other content, so a
//    later identical prefix can still revive it.
#include <stdint.h>
#include <string.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "hpkv.h"

namespace {

// ---- XXH64, written from the xxHash specification (64-bit variant) ---------
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kP3 = 0x165667B19E3779F9ull;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t read64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}
inline uint32_t read32(const uint8_t* p) {
  return uint32_t(p[0]) | uint32_t(p[1]) << 8 | uint32_t(p[2]) << 16 | uint32_t(p[3]) << 24;
}
inline uint64_t xround(uint64_t acc, uint64_t lane) { return rotl(acc + lane * kP2, 31) * kP1; }
inline uint64_t merge(uint64_t acc, uint64_t v) { return (acc ^ xround(0, v)) * kP1 + kP4; }

uint64_t xxh64(const uint8_t* p, size_t len, uint64_t seed) {
  const uint8_t* end = p + len;
  uint64_t acc;
  if (len >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    for (; p + 32 <= end; p += 32) {
      v1 = xround(v1, read64(p));
      v2 = xround(v2, read64(p + 8));
      v3 = xround(v3, read64(p + 16));
      v4 = xround(v4, read64(p + 24));
    }
    acc = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    acc = merge(acc, v1);
    acc = merge(acc, v2);
    acc = merge(acc, v3);
    acc = merge(acc, v4);
  } else {
    acc = seed + kP5;
  }
  acc += uint64_t(len);
  for (; p + 8 <= end; p += 8) acc = rotl(acc ^ xround(0, read64(p)), 27) * kP1 + kP4;
  if (p + 4 <= end) {
    acc = rotl(acc ^ (uint64_t(read32(p)) * kP1), 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) acc = rotl(acc ^ (uint64_t(*p) * kP5), 11) * kP1;
  acc ^= acc >> 33;
  acc *= kP2;
  acc ^= acc >> 29;
  acc *= kP3;
  acc ^= acc >> 32;
  return acc;
}

uint64_t page_hash(const int32_t* tokens, uint32_t n, uint64_t prev) {
  std::vector<uint8_t> bytes(size_t(n) * 4);
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t t = uint32_t(tokens[i]);
    for (int b = 0; b < 4; ++b) bytes[size_t(i) * 4 + b] = uint8_t(t >> (8 * b));
  }
  return xxh64(bytes.data(), bytes.size(), prev);
}

struct Page {
  uint32_t ref = 0;
  bool hashed = false;  // full and registered in the prefix cache
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // content of a hashed page (collision check)
};

struct Sequence {
  std::vector<uint64_t> pages;  // block table of the sequence
  std::vector<int32_t> tokens;  // every token id appended so far
  uint64_t last_hash = 0;       // hash of the last full page (0 before the first)
};

}  // namespace

struct hpkv_block_manager {
  uint32_t page_size;
  std::vector<Page> pages;
  // Pages with ref == 0, first-freed first. A page revived by a prefix hit
  // stays listed until popped, and is then skipped (in_free says it is taken).
  std::deque<uint64_t> free_list;
  std::vector<uint8_t> in_free;    // page is free (ref == 0)
  uint64_t nfree = 0;
  std::unordered_map<uint64_t, uint64_t> by_hash;  // prefix cache: hash -> page
  std::unordered_map<uint64_t, Sequence> seqs;

  // A page for new content: the oldest free page, dropped from the prefix cache.
  bool take_free(uint64_t* out) {
    while (!free_list.empty()) {
      const uint64_t p = free_list.front();
      free_list.pop_front();
      if (!in_free[p]) continue;  // revived by a prefix hit since it was freed
      in_free[p] = 0;
      --nfree;
      Page& pg = pages[p];
      if (pg.hashed) {
        auto it = by_hash.find(pg.hash);
        if (it != by_hash.end() && it->second == p) by_hash.erase(it);
        pg.hashed = false;
        pg.tokens.clear();
      }
      pg.ref = 1;
      *out = p;
      return true;
    }
    return false;
  }

  void release_page(uint64_t p) {
    if (--pages[p].ref == 0) {
      in_free[p] = 1;
      ++nfree;
      free_list.push_back(p);
    }
  }

  uint64_t num_free() const { return nfree; }

  // Registers the sequence's page `i` (now full) in the prefix cache.
  void seal(Sequence& s, uint64_t i) {
    const int32_t* t = s.tokens.data() + i * page_size;
    const uint64_t h = page_hash(t, page_size, s.last_hash);
    s.last_hash = h;
    Page& pg = pages[s.pages[i]];
    if (pg.hashed) return;
    pg.hashed = true;
    pg.hash = h;
    pg.tokens.assign(t, t + page_size);
    by_hash.emplace(h, s.pages[i]);  // an existing entry for h keeps priority
  }
};

extern "C" {

hpkv_block_manager* hpkv_bm_create(uint64_t num_pages, uint32_t page_size) {
  if (num_pages == 0 || page_size == 0) return nullptr;
  hpkv_block_manager* bm = new (std::nothrow) hpkv_block_manager();
  if (!bm) return nullptr;
  try {
    bm->page_size = page_size;
    bm->pages.resize(num_pages);
    bm->in_free.assign(num_pages, 1);
    bm->nfree = num_pages;
    for (uint64_t p = 0; p < num_pages; ++p) bm->free_list.push_back(p);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void hpkv_bm_destroy(hpkv_block_manager* bm) { delete bm; }

int hpkv_bm_admit(hpkv_block_manager* bm, uint64_t seq_id, const int32_t* token_ids,
                  uint64_t num_tokens, uint64_t* cached_tokens) {
  if (!bm || (num_tokens > 0 && !token_ids)) return HPKV_ERR_NULL;
  if (bm->seqs.count(seq_id)) return HPKV_ERR_INVALID_ARG;
  const uint32_t bs = bm->page_size;
  const uint64_t need = (num_tokens + bs - 1) / bs;
  const uint64_t full = num_tokens / bs;
  // prefix hits: leading full pages whose chained hash and tokens match
  std::vector<uint64_t> hits;
  uint64_t h = 0;
  for (uint64_t i = 0; i < full; ++i) {
    const int32_t* t = token_ids + i * bs;
    h = page_hash(t, bs, h);
    auto it = bm->by_hash.find(h);
    if (it == bm->by_hash.end()) break;
    const Page& pg = bm->pages[it->second];
    if (!pg.hashed || memcmp(pg.tokens.data(), t, size_t(bs) * 4) != 0) break;
    hits.push_back(it->second);
  }
  // capacity: fresh pages come from free pages that are not among the hits
  uint64_t revived = 0;
  for (uint64_t p : hits) revived += bm->pages[p].ref == 0;
  if (need - hits.size() > bm->num_free() - revived) return HPKV_ERR_INVALID_INDEX;
  Sequence s;
  for (uint64_t p : hits) {
    Page& pg = bm->pages[p];
    if (pg.ref++ == 0) {  // revived from the free pool
      bm->in_free[p] = 0;
      --bm->nfree;
    }
    s.pages.push_back(p);
  }
  s.tokens.assign(token_ids, token_ids + num_tokens);
  for (uint64_t i = hits.size(); i < need; ++i) {
    uint64_t p = 0;
    bm->take_free(&p);  // cannot fail: counted above
    s.pages.push_back(p);
  }
  s.last_hash = 0;
  for (uint64_t i = 0; i < full; ++i) bm->seal(s, i);
  if (cached_tokens) *cached_tokens = uint64_t(hits.size()) * bs;
  bm->seqs.emplace(seq_id, std::move(s));
  return HPKV_OK;
}

int hpkv_bm_append(hpkv_block_manager* bm, uint64_t seq_id, int32_t token_id, int64_t* slot) {
  if (!bm) return HPKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return HPKV_ERR_INVALID_ARG;
  Sequence& s = it->second;
  const uint32_t bs = bm->page_size;
  const uint64_t len = s.tokens.size() + 1;  // length after this token
  if (len % bs == 1 || bs == 1) {              // the new token opens a page
    uint64_t p = 0;
    if (!bm->take_free(&p)) return HPKV_ERR_INVALID_INDEX;
    s.pages.push_back(p);
  }
  s.tokens.push_back(token_id);
  const uint64_t pos = len - 1;
  if (slot) *slot = int64_t(s.pages[pos / bs] * bs + pos % bs);
  if (len % bs == 0) bm->seal(s, len / bs - 1);
  return HPKV_OK;
}

int hpkv_bm_release(hpkv_block_manager* bm, uint64_t seq_id) {
  if (!bm) return HPKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return HPKV_ERR_INVALID_ARG;
  // later pages first, so a revival of the prefix finds its first pages freed last
  for (auto p = it->second.pages.rbegin(); p != it->second.pages.rend(); ++p)
    bm->release_page(*p);
  bm->seqs.erase(it);
  return HPKV_OK;
}

int hpkv_bm_stats(const hpkv_block_manager* bm, uint64_t* free_pages, uint64_t* allocated_pages,
                  uint64_t* live_sequences, uint64_t* cached_pages) {
  if (!bm) return HPKV_ERR_NULL;
  const uint64_t f = bm->num_free();
  if (free_pages) *free_pages = f;
  if (allocated_pages) *allocated_pages = bm->pages.size() - f;
  if (live_sequences) *live_sequences = bm->seqs.size();
  if (cached_pages) *cached_pages = bm->by_hash.size();
  return HPKV_OK;
}

int hpkv_bm_export(const hpkv_block_manager* bm, const uint64_t* seq_ids, uint32_t num_seqs,
                   int index_type, void* block_table, uint64_t capacity, void* seq_ptr,
                   int32_t* context_lens, uint64_t* block_table_len) {
  if (!bm || (num_seqs > 0 && !seq_ids) || !seq_ptr || !block_table_len) return HPKV_ERR_NULL;
  if (index_type != HPKV_INDEX_U32 && index_type != HPKV_INDEX_U64) return HPKV_ERR_INVALID_ARG;
  if (index_type == HPKV_INDEX_U32 && bm->pages.size() > 0xffffffffull)
    return HPKV_ERR_UNSUPPORTED;
  uint64_t total = 0;
  for (uint32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return HPKV_ERR_INVALID_ARG;
    if (context_lens && it->second.tokens.size() > 0x7fffffffull) return HPKV_ERR_UNSUPPORTED;
    total += it->second.pages.size();
  }
  *block_table_len = total;
  if (total > capacity) return HPKV_ERR_WORKSPACE;
  if (total > 0 && !block_table) return HPKV_ERR_NULL;
  auto put = [&](void* base, uint64_t i, uint64_t v) {
    if (index_type == HPKV_INDEX_U64) {
      static_cast<uint64_t*>(base)[i] = v;
    } else {
      static_cast<uint32_t*>(base)[i] = uint32_t(v);
    }
  };
  uint64_t k = 0;
  put(seq_ptr, 0, 0);
  for (uint32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    for (uint64_t p : s.pages) put(block_table, k++, p);
    put(seq_ptr, i + 1, k);
    if (context_lens) context_lens[i] = int32_t(s.tokens.size());
  }
  return HPKV_OK;
}

int hpkv_bm_check(const hpkv_block_manager* bm) {
  if (!bm) return HPKV_ERR_NULL;
  const uint64_t np = bm->pages.size();
  const uint32_t bs = bm->page_size;
  std::vector<uint64_t> refs(np, 0), writers(np, 0);
  for (const auto& kv : bm->seqs) {
    const Sequence& s = kv.second;
    if (s.pages.size() != (s.tokens.size() + bs - 1) / bs) return HPKV_ERR_INVALID_INDEX;
    for (uint64_t i = 0; i < s.pages.size(); ++i) {
      if (s.pages[i] >= np) return HPKV_ERR_INVALID_INDEX;
      ++refs[s.pages[i]];
      if ((i + 1) * bs > s.tokens.size()) ++writers[s.pages[i]];  // the partial last page
    }
  }
  uint64_t free_count = 0;
  for (uint64_t p = 0; p < np; ++p) {
    const Page& pg = bm->pages[p];
    if (pg.ref != refs[p]) return HPKV_ERR_INVALID_INDEX;         // reference counts
    if (bool(bm->in_free[p]) != (pg.ref == 0)) return HPKV_ERR_INVALID_INDEX;
    free_count += bm->in_free[p];
    if (writers[p] > 0 && (refs[p] != 1 || pg.hashed)) return HPKV_ERR_INVALID_INDEX;  // alias
  }
  // free + allocated = pool, and the free list holds every free page
  uint64_t listed = 0;
  std::vector<uint8_t> seen(np, 0);
  for (uint64_t p : bm->free_list)
    if (bm->in_free[p] && !seen[p]) {
      seen[p] = 1;
      ++listed;
    }
  if (listed != free_count || free_count != bm->nfree) return HPKV_ERR_INVALID_INDEX;
  for (const auto& kv : bm->by_hash) {
    if (kv.second >= np) return HPKV_ERR_INVALID_INDEX;
    const Page& pg = bm->pages[kv.second];
    if (!pg.hashed || pg.hash != kv.first || pg.tokens.size() != bs) return HPKV_ERR_INVALID_INDEX;
  }
  return HPKV_OK;
}

uint64_t hpkv_xxh64(const void* data, uint64_t len, uint64_t seed) {
  return xxh64(static_cast<const uint8_t*>(data), size_t(len), seed);
}

}  // extern "C"
