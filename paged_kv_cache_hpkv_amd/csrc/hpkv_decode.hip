// Single-query paged decode attention for gfx950 (CDNA4).
//
// What is computed ("Paged KV Cache · AI infra interview lesson", section
// "Step 2: paged_attention_decode"): for sequence s with n context tokens and
// query head h, with KV head g = h / (Hq / Hkv),
//   out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K[t,g,:]) * V[t,g,:],
// K and V rows gathered through the CSR block table ("Block-Paged KV Cache",
// section "Element lookup through the block table").
//
// Design (HBM-bound gather; arithmetic intensity <= Hq/Hkv flop per byte):
//  * One workgroup per (sequence, head tile, context partition of part_tokens
//    tokens); a head tile is a tile of query heads of one KV head, or the
//    whole groups of two adjacent KV heads. All query heads of the tile are
//    served from one pass over the partition's K and V, so a GQA group reads
//    its KV once. The host picks the tile and the partition size per call.
//  * Kernels: the VALU kernel below (one query head per KV head, fp32, groups
//    not divisible by 4), the matrix-core kernel (16-bit GQA groups of 4+),
//    and both for quantized pools; ahead of them a one-workgroup ordering
//    pass lists the partitions longest first, and after them the reduce
//    kernel merges the partitions.
//  * The workgroup first resolves its partition through the block table into
//    an LDS table: every token's row offset (or 32-bit pool slot, on the
//    matrix-core kernel with two KV heads), or for quantized pools every
//    page's id and factors; the token loop then reads no block table.
//  * VALU kernel: a 16-byte vector load per lane; a token row of head_dim
//    elements is covered by LPR = head_dim*bytes/16 adjacent lanes, so one
//    wave load fetches RPL = 64/LPR whole rows (coalesced 2x128 B per 256 B
//    row at d=128 bf16). Each wave keeps 8 K and 8 V loads in flight per tile.
//  * q.k partial sums are reduced across the LPR lanes of a row with DPP
//    (quad_perm, row_half_mirror, row_mirror); every lane of the row then
//    holds the score, so the same lanes weight their own V chunk: no LDS
//    traffic in the token loop.
//  * Online softmax per lane group in base 2 (scores pre-multiplied by
//    scale*log2(e), v_exp_f32), fp32 accumulators; the row groups and waves
//    are merged with the log-sum-exp rule at the end of the partition.
//  * A sequence covered by one partition is normalised and written directly;
//    otherwise the partition writes (max, sum, unnormalised vector) and the
//    reduce kernel merges the partitions.
//  * Rows at or past the context length are never loaded: their lanes reuse
//    the address of the last valid row (finite data) and their score is -inf,
//    so their weight is exactly 0 and NaN garbage in unused rows cannot reach
//    the accumulators.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "hpkv_device.h"

// The build compiles this file once per part so that its kernel instantiations
// compile in parallel: part 0 holds the ordering and reduce kernels and the
// host-side launch plan, parts 1-3 the fp32, fp16 and bf16 decode kernels and
// parts 4-6 the quantized-pool kernels for fp32, fp16 and bf16 queries.
// Compiled without HPKV_DECODE_PART, one object holds every part.
#ifdef HPKV_DECODE_PART
#define HPKV_DECODE_HAS(p) (HPKV_DECODE_PART == (p))
#else
#define HPKV_DECODE_HAS(p) 1
#endif

namespace hpkv {

hipError_t launch_decode_f32(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                             hipStream_t stream);
hipError_t launch_decode_f16(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                             hipStream_t stream);
hipError_t launch_decode_bf16(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                              hipStream_t stream);
hipError_t launch_decode_quant_f32(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                   uint64_t nwg, hipStream_t stream);
hipError_t launch_decode_quant_f16(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                   uint64_t nwg, hipStream_t stream);
hipError_t launch_decode_quant_bf16(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                    uint64_t nwg, hipStream_t stream);

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                // waves per workgroup of the reduce kernel
constexpr int kThreads = kWave * kWaves;

// Launch shape of the partition kernel: waves per workgroup, token rows each
// lane loads per tile (NLOAD, each row CPL 16-byte chunks of K and of V),
// non-temporal loads, the minimum waves per SIMD the register budget must
// allow, and CPL, the 16-byte chunks of a row one lane owns. A larger CPL
// puts fewer lanes on a row, so the per-token softmax bookkeeping and the
// cross-lane reduction of q.k are repeated on fewer lanes.
template <int NW_, int NLOAD_, bool NT_, int MINW_, int CPL_ = 1>
struct Tune {
  static constexpr int NW = NW_;
  static constexpr int NLOAD = NLOAD_;
  static constexpr bool NT = NT_;
  static constexpr int MINW = MINW_;
  static constexpr int CPL = CPL_;
};

// fp32 dot product of one 16-byte chunk of K with the matching chunk of q.
template <int DT>
__device__ inline float dot16(const u32x4 k, const u32x4 q) {
  const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float a = 0.0f;
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a = __builtin_amdgcn_fdot2_f32_bf16(as_pair<bf16x2>(kw[i]), as_pair<bf16x2>(qw[i]), a,
                                          false);
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a = __builtin_amdgcn_fdot2(as_pair<f16x2>(kw[i]), as_pair<f16x2>(qw[i]), a, false);
  } else {
    a = __uint_as_float(kw[0]) * __uint_as_float(qw[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) a = fmaf(__uint_as_float(kw[i]), __uint_as_float(qw[i]), a);
  }
  return a;
}

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPR adjacent lanes that hold one token row; every lane of the
// group receives the total.
template <int LPR>
__device__ inline float row_sum(float x) {
  if constexpr (LPR >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
  return x;
}

// The sequence-level checks the reduce kernel can also make (it sees only
// context_lens): a negative length or one above max_context_len.
__device__ inline bool length_is_bad(int32_t n, uint32_t max_context_len) {
  return n < 0 || uint32_t(n) > max_context_len;
}

__device__ inline uint32_t num_parts(int32_t n, uint32_t part_tokens) {
  return n <= 0 ? 1u : (uint32_t(n) + part_tokens - 1) / part_tokens;
}

// Workgroup-level description of one partition's work.
struct Partition {
  uint32_t s;          // sequence
  uint32_t g;          // KV head
  uint32_t part;       // partition index within the sequence
  uint32_t nparts;     // partitions of the sequence
  uint32_t cnt;        // tokens of this partition
  uint64_t out_row0;   // first (sequence, query head) row of the head tile
};

// One work item: sequence, partition, KV head g and the first query head h0
// of the tile it serves, and the sequences s .. s+members-1 it serves (more
// than one for a shared run). s == kNoWork: the item does nothing.
struct WorkItem {
  uint32_t s, part, g, h0, members;
};

// Order-list entry (and WorkItem::s) of a pair with nothing to do: a partition
// past its sequence's context, or not the first partition of a malformed
// length. Such workgroups exit before reading anything else.
constexpr uint32_t kNoWork = 0xffffffffu;

// Grid order: head tile fastest, then the (sequence, partition) pair. A head
// tile is GT query heads of one KV head, or the whole groups of kv_per_wg
// adjacent KV heads. The pairs are taken from the ordering pass's list
// (longest partitions first, see below) when it ran, else in partition-major
// order (every sequence has a partition 0, so the first num_seqs*head_tiles
// workgroups all carry work). Tile ht serves query heads [h0, h0 + GT) of KV
// head g.
// With fewer head tiles than the 8 XCDs (T = head_tiles dividing 8), workgroups
// dispatched round-robin over the XCDs would alternate consecutive sequences
// between the R = 8/T XCDs that serve one head tile. CHUNKED remaps the block
// index so that each of those XCDs takes runs of kXcdChunk consecutive
// (sequence, partition) items instead: neighbouring sequences that alias the
// same prefix pages then read them through one XCD's L2. The remap is a
// bijection on the largest multiple of 8*kXcdChunk blocks; the rest keep
// their index.
constexpr uint32_t kXcdChunk = 16;

template <int GT, bool CHUNKED = false>
__device__ inline WorkItem grid_item(const DecodeKernelArgs& a) {
  uint32_t bid = blockIdx.x;
  if constexpr (CHUNKED) {
    const uint32_t T = a.head_tiles;
    if (T < 8 && 8 % T == 0) {
      const uint32_t R = 8 / T;
      const uint32_t full = gridDim.x / (8 * kXcdChunk) * (8 * kXcdChunk);
      if (bid < full) {
        const uint32_t x = bid % 8, j = bid / 8;  // XCD, and the block's turn on it
        const uint32_t q = (j / kXcdChunk) * (R * kXcdChunk) + (x / T) * kXcdChunk +
                           j % kXcdChunk;       // (sequence, partition) item
        bid = x % T + T * q;
      }
    }
  }
  const uint32_t ht = bid % a.head_tiles;
  bid /= a.head_tiles;  // (sequence, partition) pair, partition-major
  WorkItem it;
  it.members = 1;
  if (a.order != nullptr) {
    bid = a.order[bid];
    if (bid == kNoWork) {
      it.s = kNoWork;
      it.part = it.g = it.h0 = 0;
      return it;
    }
    if (a.share_block > 1) {
      it.members = (bid >> kRunShift) + 1;
      bid &= kPairMask;
    }
  }
  it.s = bid % a.num_seqs;
  it.part = bid / a.num_seqs;
  const uint32_t tiles_per_group = a.group / GT;  // 1 when kv_per_wg > 1
  it.g = (ht / tiles_per_group) * a.kv_per_wg;
  it.h0 = it.g * a.group + (ht % tiles_per_group) * GT;
  return it;
}

// Longest-first dispatch of the split-context work. A launch in which
// partitions of every length (full ones of long contexts, short tails, short
// contexts) are dispatched in partition-major order ends with a few long
// workgroups still running on a mostly idle chip. The ordering pass sorts
// the (sequence, partition) pairs j = s + num_seqs * part by the length of
// their partition, longest first (list scheduling with the longest jobs first,
// which bounds that tail by the shortest jobs): 17 classes, full partitions,
// then 16 bands of partial ones from long to short, then empty pairs (past the
// context, or of a malformed length). The sort is stable, so within a class
// the pairs keep the partition-major order and the XCD placement above. One
// workgroup: wave w sorts the contiguous slice w of the pairs in a count pass
// and a scatter pass that ranks each pair among its class with a ballot,
// between them an exclusive scan over (class, wave) in LDS.
constexpr int kOrderWaves = 16;
constexpr uint32_t kOrderClasses = 17;
constexpr uint32_t kOrderLdsSeqs = 8192;  // batches up to this size read lengths from LDS

__device__ inline uint32_t order_class(const DecodeKernelArgs& a, const int32_t* lens,
                                       uint32_t j) {
  if (a.share_flags != nullptr && a.share_flags[j]) return kOrderClasses - 1;  // a follower
  const uint32_t s = j % a.num_seqs, part = j / a.num_seqs;
  const int32_t n = lens[s];
  const uint32_t p0 = part * a.part_tokens;  // < max_context_len + part_tokens < 2^32
  if (n <= 0 || uint32_t(n) > a.max_context_len || uint32_t(n) <= p0) return kOrderClasses - 1;
  const uint32_t len = min(uint32_t(n) - p0, a.part_tokens);
  return (a.part_tokens - len) * 16u / a.part_tokens;  // 0 (full) .. 15
}

#if HPKV_DECODE_HAS(0)
// Shared partitions ("Block-Paged KV Cache", "Element lookup through the block
// table": sequences that alias the same pages read the same K/V rows). One wave
// per (sequence, partition) pair j = s + B*part: the flag is 1 when s is not the
// first of its aligned block of share_block sequences, both s and s - 1 have a
// valid length and slice, partition `part` is full for both, and every page id
// of that partition (at most kSharePagesMax pages) is the same, inside the pool,
// in both tables. Then the two read exactly the same rows for that partition.
constexpr uint32_t kSharePagesMax = 256;
constexpr int kShareWaves = 4;

__global__ __launch_bounds__(kShareWaves * kWave) void decode_share_kernel(
    const DecodeKernelArgs a) {
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t j = blockIdx.x * kShareWaves + threadIdx.x / kWave;
  if (j >= a.num_seqs * a.max_parts) return;
  const uint32_t s = j % a.num_seqs, part = j / a.num_seqs;
  bool same = false;
  if (s % a.share_block != 0) {
    const uint32_t P = a.part_tokens, p0 = part * P;
    const int32_t n1 = a.context_lens[s], n0 = a.context_lens[s - 1];
    const uint64_t f1 = read_idx(a.seq_ptr, s, a.idx64);
    const uint64_t l1 = read_idx(a.seq_ptr, uint64_t(s) + 1, a.idx64);
    const uint64_t f0 = read_idx(a.seq_ptr, s - 1, a.idx64);
    auto full = [&](int32_t n, uint64_t f, uint64_t l) {
      return !length_is_bad(n, a.max_context_len) && uint32_t(n) >= p0 + P && f <= l &&
             l <= a.block_table_len && uint64_t(n) <= (l - f) * uint64_t(a.page_size);
    };
    const uint32_t k0 = fastdiv(p0, a.page_div), k1 = fastdiv(p0 + P - 1, a.page_div);
    const uint32_t npp = k1 - k0 + 1;
    // s - 1's slice ends where s's begins (CSR), so f0 <= l0 == f1
    if (full(n1, f1, l1) && full(n0, f0, f1) && npp <= kSharePagesMax) {
      bool eq = true;
      for (uint32_t k = lane; k < npp; k += kWave) {
        const uint64_t a1 = read_idx(a.block_table, f1 + k0 + k, a.idx64);
        const uint64_t a0 = read_idx(a.block_table, f0 + k0 + k, a.idx64);
        eq = eq && a1 == a0 && a1 < a.num_pages;
      }
      same = __all(eq);
    }
  }
  if (lane == 0) a.share_flags[j] = same ? 1 : 0;
}

hipError_t launch_share(const DecodeKernelArgs& a, hipStream_t stream) {
  if (a.share_flags == nullptr) return hipSuccess;
  const uint32_t pairs = a.num_seqs * a.max_parts;
  hipLaunchKernelGGL(decode_share_kernel, dim3((pairs + kShareWaves - 1) / kShareWaves),
                     dim3(kShareWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(kOrderWaves * kWave) void decode_order_kernel(
    const DecodeKernelArgs a) {
  __shared__ uint32_t s_cnt[kOrderClasses][kOrderWaves];
  __shared__ int32_t s_len[kOrderLdsSeqs];
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t n = a.num_seqs * a.max_parts;
  // the lengths are read once per pair in each pass: stage them in LDS
  const int32_t* lens = a.context_lens;
  if (a.num_seqs <= kOrderLdsSeqs) {
    for (uint32_t i = threadIdx.x; i < a.num_seqs; i += kOrderWaves * kWave)
      s_len[i] = a.context_lens[i];
    __syncthreads();
    lens = s_len;
  }
  const uint32_t per = ((n + kOrderWaves - 1) / kOrderWaves + kWave - 1) / kWave * kWave;
  const uint32_t lo = min(n, wave * per), hi = min(n, lo + per);

  uint32_t cnt[kOrderClasses];
#pragma unroll
  for (uint32_t k = 0; k < kOrderClasses; ++k) cnt[k] = 0;
  for (uint32_t j0 = lo; j0 < hi; j0 += kWave) {
    const uint32_t j = j0 + lane;
    const uint32_t c = j < hi ? order_class(a, lens, j) : kOrderClasses;
#pragma unroll
    for (uint32_t k = 0; k < kOrderClasses; ++k) cnt[k] += __popcll(__ballot(c == k));
  }
  if (lane == 0) {
#pragma unroll
    for (uint32_t k = 0; k < kOrderClasses; ++k) s_cnt[k][wave] = cnt[k];
  }
  __syncthreads();

  // First position of (class k, this wave): every pair of the classes before
  // k, then the pairs of class k in the slices before this one. Lane k < 17
  // sums its class over the waves; an exclusive scan over those lanes adds
  // the classes before it.
  uint32_t before = 0, total = 0;
  if (lane < kOrderClasses) {
    for (uint32_t v = 0; v < uint32_t(kOrderWaves); ++v) {
      const uint32_t c = s_cnt[lane][v];
      total += c;
      before += v < wave ? c : 0u;
    }
  }
  uint32_t incl = total;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= uint32_t(o)) incl += t;
  }
  const uint32_t start = incl - total + before;
  uint32_t base[kOrderClasses];
#pragma unroll
  for (uint32_t k = 0; k < kOrderClasses; ++k) base[k] = __builtin_amdgcn_readlane(start, k);
  const uint64_t below = (uint64_t(1) << lane) - 1;  // lanes before this one
  for (uint32_t j0 = lo; j0 < hi; j0 += kWave) {
    const uint32_t j = j0 + lane;
    const uint32_t c = j < hi ? order_class(a, lens, j) : kOrderClasses;
    uint32_t pos = n;
#pragma unroll
    for (uint32_t k = 0; k < kOrderClasses; ++k) {
      const uint64_t m = __ballot(c == k);
      if (c == k) pos = base[k] + uint32_t(__popcll(m & below));
      base[k] += uint32_t(__popcll(m));
    }
    // pairs past a context (or after the first of a malformed length) and the
    // followers of shared runs do nothing: their workgroups need not even read the
    // length; the first pair of a run carries the run's length
    if (pos < n) {
      uint32_t e = c == kOrderClasses - 1 && j >= a.num_seqs ? kNoWork : j;
      if (a.share_flags != nullptr && c < kOrderClasses) {
        if (a.share_flags[j]) {
          e = kNoWork;
        } else if (c < kOrderClasses - 1) {
          const uint32_t s = j % a.num_seqs;
          uint32_t k = 1;
          while (k < a.share_block && (s + k) % a.share_block != 0 && s + k < a.num_seqs &&
                 a.share_flags[j + k])
            ++k;
          e = j | ((k - 1) << kRunShift);
        }
      }
      a.order[pos] = e;
    }
  }
}

hipError_t launch_order(const DecodeKernelArgs& a, hipStream_t stream) {
  if (a.order == nullptr) return hipSuccess;
  const hipError_t e = launch_share(a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderWaves * kWave), 0, stream, a);
  return hipGetLastError();
}
#endif  // HPKV_DECODE_HAS(0)

// Checks the item's sequence length and table slice, and resolves each token
// of the partition to the element offset of head g's row in the pool (s_row);
// a workgroup serving NKV adjacent KV heads g .. g+NKV-1 finds head g+i's row
// i*D elements further. Returns false when the workgroup has nothing (more) to
// do; for a malformed sequence it has then already written the NaN result of
// its NH query heads h0 .. h0+NH-1.
// No per-token work beyond the row table.
struct NoTokenHook {
  __device__ void operator()(uint32_t, uint64_t) const {}
};

// The checks every workgroup makes before it resolves its rows: no-work entry,
// partition past the context, malformed length (its NaN result is written here),
// malformed table slice or a partition longer than the row table holds
// (`fits` false; reported through `bad`). Fills w (w.cnt = 0 when bad).
template <int DT, int D, int NH, int NTH>
__device__ inline bool begin_partition(const DecodeKernelArgs& a, const WorkItem& it, bool fits,
                                       Partition& w, uint64_t& first, bool& bad,
                                       bool& slot_writer) {
  if (it.s == kNoWork) return false;
  const uint32_t tid = threadIdx.x;
  w.s = it.s;
  w.part = it.part;
  w.g = it.g;
  const uint32_t h0 = it.h0;

  // the length and the table slice bounds are independent loads: issue both
  const int32_t n = a.context_lens[w.s];
  first = read_idx(a.seq_ptr, w.s, a.idx64);
  const uint64_t last = read_idx(a.seq_ptr, uint64_t(w.s) + 1, a.idx64);
  w.nparts = num_parts(n, a.part_tokens);
  if (w.part >= w.nparts) return false;

  w.out_row0 = uint64_t(w.s) * a.num_q_heads + h0;
  slot_writer = a.slots_out != nullptr && tid == 0 && h0 == 0;  // once per sequence
  if (length_is_bad(n, a.max_context_len)) {
    if (w.part == 0) {
      for (uint32_t i = tid; i < NH * D; i += NTH) store_out<DT>(a.out, w.out_row0 * D + i, NAN);
      if (slot_writer) a.slots_out[w.s] = -1;
    }
    return false;
  }

  // (a partition longer than the row table cannot come from the host's plan; it is
  // refused here rather than written past the table)
  bad = first > last || last > a.block_table_len ||
        uint64_t(n) > (last - first) * uint64_t(a.page_size) || !fits;
  const uint32_t p0 = w.part * a.part_tokens;
  w.cnt = bad || n == 0 ? 0u : min(uint32_t(n) - p0, a.part_tokens);
  return true;
}

// Malformed index buffers: NaN result (or NaN partials) for this partition.
template <int DT, int D, int NH, int NTH>
__device__ inline void fail_partition(const DecodeKernelArgs& a, const Partition& w,
                                      bool slot_writer) {
  const uint32_t tid = threadIdx.x;
  if (w.nparts == 1) {
    for (uint32_t i = tid; i < NH * D; i += NTH) store_out<DT>(a.out, w.out_row0 * D + i, NAN);
  } else {
    for (uint32_t i = tid; i < NH * D; i += NTH) {
      const uint64_t r = (w.out_row0 + i / D) * a.max_parts + w.part;
      a.ws_o[r * D + i % D] = NAN;
      if (i % D == 0) a.ws_ml[r] = make_float2(NAN, NAN);
    }
  }
  if (slot_writer && w.part + 1 == w.nparts) a.slots_out[w.s] = -1;
}

template <int DT, int D, int NH, int NTH, class Hook = NoTokenHook, int NKV = 1,
          class RowT = uint64_t, uint32_t CAP = 0>
__device__ inline bool setup_partition(const DecodeKernelArgs& a, const WorkItem& it,
                                       RowT (&s_row)[CAP], Partition& w,
                                       Hook on_token = Hook{}) {
  // 64-bit entries hold element offsets; 32-bit entries hold the token's pool slot
  // (the host takes a shape with them only for pools of at most 2^32 slots)
  constexpr bool kSlots = sizeof(RowT) == 4;
  const uint32_t tid = threadIdx.x;
  uint64_t first = 0;
  bool bad = false, slot_writer = false;
  if (!begin_partition<DT, D, NH, NTH>(a, it, a.part_tokens <= CAP, w, first, bad, slot_writer))
    return false;
  const uint32_t p0 = w.part * a.part_tokens;

  // Each thread resolves tokens tid, tid + NTH, ...: all of its table reads are
  // issued before the first is used, so the table costs one memory round trip.
  constexpr uint32_t KT = (CAP + NTH - 1) / NTH;
  uint64_t phys[KT];
#pragma unroll
  for (uint32_t k = 0; k < KT; ++k) {
    const uint32_t i = tid + k * NTH;
    phys[k] = i < w.cnt ? read_idx(a.block_table, first + fastdiv(p0 + i, a.page_div), a.idx64)
                        : 0;
  }
  int bad_page = 0;
#pragma unroll
  for (uint32_t k = 0; k < KT; ++k) {
    const uint32_t i = tid + k * NTH;
    if (i < w.cnt) {
      const uint32_t t = p0 + i;
      const uint32_t off = t - fastdiv(t, a.page_div) * a.page_size;
      uint64_t ph = phys[k];
      if (ph >= a.num_pages) {
        bad_page = 1;
        ph = 0;
      }
      const uint64_t slot = ph * a.page_size + off;
      s_row[i] = kSlots ? RowT(slot) : RowT((slot * a.num_kv_heads + w.g) * uint64_t(D));
      on_token(i, ph);
    }
  }
  bad = __syncthreads_or(bad_page) != 0 || bad;

  const bool last_part = w.part + 1 == w.nparts;
  if (bad) {
    fail_partition<DT, D, NH, NTH>(a, w, slot_writer);
    return false;
  }

  // Fused decode step ("Paged KV Cache · AI infra interview lesson", Step 1
  // store at the decode slot p = ctx-1, then Step 2): the workgroup whose
  // partition ends the context first writes the new token's K and V rows of
  // its heads g .. g+NKV-1 (adjacent in the new rows and in the pool row) to
  // that token's pool row (its offset is already in s_row), and the barrier
  // makes them visible to the workgroup's own loads below.
  if (a.new_k != nullptr && last_part) {
    if (w.cnt > 0) {
      constexpr int EB = Elem<DT>::bytes;
      constexpr int CH = NKV * D * EB / 16;  // 16-byte chunks of the heads' rows
      const uint64_t last_row =
          kSlots ? (uint64_t(s_row[w.cnt - 1]) * a.num_kv_heads + w.g) * uint64_t(D)
                 : uint64_t(s_row[w.cnt - 1]);  // element offset of the token's row
      const uint64_t dst = last_row * EB;
      const uint64_t src = (uint64_t(w.s) * a.num_kv_heads + w.g) * D * EB;
      for (uint32_t i = tid; i < uint32_t(CH); i += NTH) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.new_k) + src + i * 16);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.new_v) + src + i * 16);
        *reinterpret_cast<u32x4*>(const_cast<char*>(static_cast<const char*>(a.k_cache)) + dst + i * 16) = kv;
        *reinterpret_cast<u32x4*>(const_cast<char*>(static_cast<const char*>(a.v_cache)) + dst + i * 16) = vv;
      }
      if (slot_writer) {
        const uint64_t row = last_row / D;  // (slot * Hkv + g)
        a.slots_out[w.s] = int64_t((row - w.g) / a.num_kv_heads);
      }
      __syncthreads();
    } else if (slot_writer) {
      a.slots_out[w.s] = -1;  // empty context: nothing appended
    }
  }
  return true;
}

// Quantized pools: the row table is kept per page instead of per token (the
// page factors are per page and KV head anyway), so a partition of up to
// kQuantTablePages pages fits: 512 tokens of 1-token pages, 2048 tokens of pages
// of 4 or more. Entry k of s_page is the pool page of the partition's k-th page,
// k = fastdiv(p) - k0 for the token at position p, and s_fac[k][h] holds that
// page's (k scale, k zero + bias, v scale, v zero + bias) for KV head g + h.
// Same checks and malformed-input results as setup_partition; no fused store.
template <int DT, int D, int NH, int NTH, int NKV, uint32_t CAPP>
__device__ inline bool setup_pages(const DecodeKernelArgs& a, const WorkItem& it, float bias,
                                   float vbias, uint32_t (&s_page)[CAPP], float4 (&s_fac)[CAPP][NKV],
                                   Partition& w, uint32_t& k0) {
  const uint32_t tid = threadIdx.x;
  uint64_t first = 0;
  bool bad = false, slot_writer = false;
  if (!begin_partition<DT, D, NH, NTH>(a, it, true, w, first, bad, slot_writer)) return false;
  const uint32_t p0 = w.part * a.part_tokens;
  k0 = fastdiv(p0, a.page_div);
  uint32_t npg = w.cnt == 0 ? 0u : fastdiv(p0 + w.cnt - 1, a.page_div) - k0 + 1;
  if (npg > CAPP) {  // not from the host's plan: refused rather than written past the table
    bad = true;
    npg = 0;
  }
  constexpr uint32_t KP = (CAPP + NTH - 1) / NTH;
  uint64_t phys[KP];
#pragma unroll
  for (uint32_t k = 0; k < KP; ++k) {
    const uint32_t i = tid + k * NTH;
    phys[k] = i < npg ? read_idx(a.block_table, first + k0 + i, a.idx64) : 0;
  }
  int bad_page = 0;
#pragma unroll
  for (uint32_t k = 0; k < KP; ++k) {
    const uint32_t i = tid + k * NTH;
    if (i < npg) {
      uint64_t ph = phys[k];
      if (ph >= a.num_pages) {
        bad_page = 1;
        ph = 0;
      }
      s_page[i] = uint32_t(ph);  // num_pages * Hkv < 2^32 for quantized pools
#pragma unroll
      for (int h = 0; h < NKV; ++h) {
        const uint64_t f = ph * a.num_kv_heads + w.g + h;
        s_fac[i][h] = make_float4(a.k_scale[f], a.k_zero[f] + bias, a.v_scale[f],
                                  a.v_zero[f] + vbias);
      }
    }
  }
  bad = __syncthreads_or(bad_page) != 0 || bad;
  if (bad) {
    fail_partition<DT, D, NH, NTH>(a, w, slot_writer);
    return false;
  }
  return true;
}

// Merges the waves' (max, sum, vector) triples for each query head of the
// tile (log-sum-exp rule) and writes the normalised result, or the partial of
// this partition when the sequence has several. With HPW KV heads per
// workgroup, wave v serves head v % HPW and the query heads of KV head i
// follow those of head i-1 in the output.
template <int DT, int D, int GT, int NW, int HPW = 1>
__device__ inline void finish_partition(const DecodeKernelArgs& a, const Partition& w,
                                        const float (*s_m)[GT], const float (*s_l)[GT],
                                        const float (*s_acc)[GT][D]) {
  constexpr int SPLIT = NW / HPW;  // waves per KV head
  for (uint32_t i = threadIdx.x; i < HPW * GT * D; i += NW * kWave) {
    const uint32_t hw = i / (GT * D), hh = (i / D) % GT, e = i % D;
    float mx = s_m[hw][hh];
#pragma unroll
    for (int v = 1; v < SPLIT; ++v) mx = fmaxf(mx, s_m[v * HPW + hw][hh]);
    const float mref = mx == -INFINITY ? 0.0f : mx;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int v = 0; v < SPLIT; ++v) {
      const float f = __builtin_amdgcn_exp2f(s_m[v * HPW + hw][hh] - mref);
      L = fmaf(s_l[v * HPW + hw][hh], f, L);
      O = fmaf(s_acc[v * HPW + hw][hh][e], f, O);
    }
    const uint64_t row = w.out_row0 + hw * GT + hh;
    if (w.nparts == 1) {
      store_out<DT>(a.out, row * D + e, L > 0.0f ? O / L : 0.0f);
    } else {
      const uint64_t r = row * a.max_parts + w.part;
      a.ws_o[r * D + e] = O;
      if (e == 0) a.ws_ml[r] = make_float2(mx, L);
    }
  }
}

// HPW adjacent KV heads per workgroup (whole GQA groups, GT == group): a token's
// rows of those heads are HPW*D contiguous elements, read as one row by HPW*LPH
// lanes; each aligned group of LPH lanes holds one head (lane head hw) and keeps
// that head's softmax state. The query heads of the workgroup are contiguous.
template <int DT, int D, int GT, class TU, int HPW>
__global__ __launch_bounds__(TU::NW * 64, TU::MINW) void decode_partition_kernel(
    const DecodeKernelArgs a) {
  constexpr int NW = TU::NW;
  constexpr int NTH = NW * kWave;    // threads per workgroup
  constexpr int NLOAD = TU::NLOAD;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int EPL = 16 / EB;       // elements per 16-byte chunk
  constexpr int CPR = D / EPL;       // chunks per token row
  constexpr int CPL = TU::CPL < CPR ? TU::CPL : CPR;  // chunks per lane
  constexpr int LPH = CPR / CPL;     // lanes per head row
  constexpr int LPR = HPW * LPH;     // lanes per token row (the workgroup's heads)
  constexpr int RPL = kWave / LPR;   // token rows per wave load
  constexpr int TT = RPL * NLOAD;    // tokens per wave tile
  constexpr int VPL = CPL * EPL;     // elements of a row per lane
  constexpr int GW = HPW * GT;       // query heads of the workgroup
  static_assert(CPR % CPL == 0 && LPR <= kWave && (LPH & (LPH - 1)) == 0 &&
                    (HPW & (HPW - 1)) == 0,
                "unsupported head_dim");

  __shared__ uint64_t s_row[kLongPartTokens];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ float s_acc[NW][GW][D];

  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = threadIdx.x / kWave;
  Partition w;
  if (!setup_partition<DT, D, GW, NTH, NoTokenHook, HPW>(a, grid_item<GT>(a), s_row, w)) return;
  const uint32_t cnt = w.cnt;
  const uint64_t out_row0 = w.out_row0;

  const uint32_t row = lane / LPR;         // which row of a wave load this lane reads
  const uint32_t hw = (lane % LPR) / LPH;  // the lane's KV head within the workgroup's
  const uint32_t c = lane % LPH;           // lane's chunks of the head row: j*LPH + c, j < CPL

  u32x4 qv[GT][CPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const char* qp = static_cast<const char*>(a.q) +
                       ((out_row0 + hw * GT + hh) * D + (j * LPH + c) * EPL) * EB;
      qv[hh][j] = *reinterpret_cast<const u32x4*>(qp);
    }
  }

  float m[GT], l[GT], acc[GT][VPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) acc[hh][e] = 0.0f;
  }

  const char* kbase = static_cast<const char*>(a.k_cache) + hw * D * EB + c * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + hw * D * EB + c * 16;

  for (uint32_t tb = wave * TT; tb < cnt; tb += NW * TT) {
    u32x4 kr[NLOAD][CPL], vr[NLOAD][CPL];
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      const uint32_t li = tb + k * RPL + row;
      const uint64_t off = s_row[li < cnt ? li : cnt - 1] * EB;
#pragma unroll
      for (int j = 0; j < CPL; ++j) kr[k][j] = load16<TU::NT>(kbase + off + j * LPH * 16);
#pragma unroll
      for (int j = 0; j < CPL; ++j) vr[k][j] = load16<TU::NT>(vbase + off + j * LPH * 16);
    }

    float sc[GT][NLOAD];
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      const bool valid = tb + k * RPL + row < cnt;
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        float part_dot = dot16<DT>(kr[k][0], qv[hh][0]);
#pragma unroll
        for (int j = 1; j < CPL; ++j) part_dot += dot16<DT>(kr[k][j], qv[hh][j]);
        const float z = row_sum<LPH>(part_dot) * a.scale_log2;
        sc[hh][k] = valid ? z : -INFINITY;
      }
    }

    float mu[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float mt = sc[hh][0];
#pragma unroll
      for (int k = 1; k < NLOAD; ++k) mt = fmaxf(mt, sc[hh][k]);
      const float mn = fmaxf(m[hh], mt);
      mu[hh] = mn == -INFINITY ? 0.0f : mn;
      const float corr = __builtin_amdgcn_exp2f(m[hh] - mu[hh]);
      l[hh] *= corr;
#pragma unroll
      for (int e = 0; e < VPL; ++e) acc[hh][e] *= corr;
      m[hh] = mn;
    }
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      float p[GT];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        p[hh] = __builtin_amdgcn_exp2f(sc[hh][k] - mu[hh]);
        l[hh] += p[hh];
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float vf[EPL];
        widen16<DT>(vr[k][j], vf);
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[hh][j * EPL + e] = fmaf(p[hh], vf[e], acc[hh][j * EPL + e]);
        }
      }
    }
  }

  // Merge the RPL row groups of the wave (log-sum-exp rule).
#pragma unroll
  for (int sh = LPR; sh < kWave; sh <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float mo = __shfl_xor(m[hh], sh);
      const float lo = __shfl_xor(l[hh], sh);
      const float mn = fmaxf(m[hh], mo);
      const float mref = mn == -INFINITY ? 0.0f : mn;
      const float fa = __builtin_amdgcn_exp2f(m[hh] - mref);
      const float fb = __builtin_amdgcn_exp2f(mo - mref);
      l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        const float ao = __shfl_xor(acc[hh][e], sh);
        acc[hh][e] = acc[hh][e] * fa + ao * fb;
      }
      m[hh] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          s_acc[wave][hw * GT + hh][(j * LPH + c) * EPL + e] = acc[hh][j * EPL + e];
      }
      if (c == 0) {
        s_m[wave][hw * GT + hh] = m[hh];
        s_l[wave][hw * GT + hh] = l[hh];
      }
    }
  }
  __syncthreads();

  finish_partition<DT, D, GW, NW>(a, w, s_m, s_l, s_acc);
}


// ---------------------------------------------------------------------------
// Quantized pools (int8 or OCP fp8 E4M3, one byte per element). Per-block-
// affine quantization with one block per page ("Block-Paged KV Cache",
// section "Quantization compatibility"): the page slot of token t carries, per
// KV head, scale and zero point for K and V, and a code c stands for
// scale * (value(c) - zero). With the page factors of token t,
//   q . k_t = ks_t * (q . value(kc_t) - kz_t * sum(q)),
//   sum_t p_t v_t = sum_t (p_t vs_t) value(vc_t) - sum_t (p_t vs_t) vz_t,
// so the inner loops work on the raw code values: one conversion and one FMA
// per element, the scales enter once per token. int8 codes are read as
// unsigned bytes of code + 128 (sign bit flipped), the 128 folded into the
// zero point. Lane layout, softmax and merges are those of the kernel above
// with 16 one-byte elements per lane chunk.
// ---------------------------------------------------------------------------

// The 16 code values of one 16-byte chunk as floats (int8: value + 128).
template <int QT>
__device__ inline void codes16(const u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (QT == kFP8) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    } else {
      const uint32_t u = w[i] ^ 0x80808080u;
      f[4 * i] = float(u & 0xffu);
      f[4 * i + 1] = float((u >> 8) & 0xffu);
      f[4 * i + 2] = float((u >> 16) & 0xffu);
      f[4 * i + 3] = float(u >> 24);
    }
  }
}

// Two exact code values (fp32) as a packed 16-bit pair of the q type.
template <int DT>
__device__ inline uint32_t pack_exact16(float x, float y) {
  if constexpr (DT == kBF16) {  // at most 8 significant bits: the upper halves are exact
    return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
  } else {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x, y);  // exact: no rounding happens
    uint32_t r;
    __builtin_memcpy(&r, &h, 4);
    return r;
  }
}

// 16 codes (one 16-byte chunk) as 16 exact 16-bit values: `lo` holds elements
// 0..7, `hi` elements 8..15.
template <int DT, int QT>
__device__ inline void codes16_to_bits16(const u32x4 c, u32x4& lo, u32x4& hi) {
  if constexpr (QT == kFP8) {  // packed scaled conversion with scale 1: exact
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == kBF16) {
        const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
        __builtin_memcpy(&r[2 * i], &a, 4);
        __builtin_memcpy(&r[2 * i + 1], &b, 4);
      } else {
        const auto a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
        const auto b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
        __builtin_memcpy(&r[2 * i], &a, 4);
        __builtin_memcpy(&r[2 * i + 1], &b, 4);
      }
    }
    lo = u32x4{r[0], r[1], r[2], r[3]};
    hi = u32x4{r[4], r[5], r[6], r[7]};
    return;
  }
  float f[16];
  codes16<QT>(c, f);
  lo = u32x4{pack_exact16<DT>(f[0], f[1]), pack_exact16<DT>(f[2], f[3]),
             pack_exact16<DT>(f[4], f[5]), pack_exact16<DT>(f[6], f[7])};
  hi = u32x4{pack_exact16<DT>(f[8], f[9]), pack_exact16<DT>(f[10], f[11]),
             pack_exact16<DT>(f[12], f[13]), pack_exact16<DT>(f[14], f[15])};
}

// Eight codes (two words) as exact 16-bit values of the q type: one operand.
template <int DT, int QT>
__device__ inline u32x4 codes8_to_bits16(const uint2 c) {
  const uint32_t w[2] = {c.x, c.y};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (QT == kFP8) {  // packed scaled conversion with scale 1: exact
      if constexpr (DT == kBF16) {
        const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
        __builtin_memcpy(&r[2 * i], &a, 4);
        __builtin_memcpy(&r[2 * i + 1], &b, 4);
      } else {
        const auto a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
        const auto b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
        __builtin_memcpy(&r[2 * i], &a, 4);
        __builtin_memcpy(&r[2 * i + 1], &b, 4);
      }
    } else {  // int8 as code + 128 (sign bit flipped): 0..255, exact in fp32 and 16 bits
      const uint32_t u = w[i] ^ 0x80808080u;
      r[2 * i] = pack_exact16<DT>(float(u & 0xffu), float((u >> 8) & 0xffu));
      r[2 * i + 1] = pack_exact16<DT>(float((u >> 16) & 0xffu), float(u >> 24));
    }
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// HPW adjacent KV heads per workgroup (whole GQA groups, GT == group): a token's
// codes of those heads are HPW*D contiguous bytes, read as one row by HPW*D/16
// lanes; each aligned group of D/16 lanes holds one head (lane head hw) and keeps
// that head's softmax state. The query heads of the workgroup are contiguous.
template <int DT, int QT, int D, int GT, class TU, int HPW>
__global__ __launch_bounds__(TU::NW * 64, TU::MINW) void decode_partition_quant_kernel(
    const DecodeKernelArgs a) {
  constexpr int NW = TU::NW;
  constexpr int NTH = NW * kWave;
  constexpr int NLOAD = TU::NLOAD;
  constexpr int EQ = Elem<DT>::bytes;  // bytes of a q / out element
  constexpr int EPL = 16;              // codes per 16-byte chunk
  constexpr int LPH = D / EPL;         // lanes per head row
  constexpr int LPR = HPW * LPH;       // lanes per token row (the workgroup's heads)
  constexpr int RPL = kWave / LPR;     // token rows per wave load
  constexpr int TT = RPL * NLOAD;      // tokens per wave tile
  constexpr int GW = HPW * GT;         // query heads of the workgroup
  static_assert(D % EPL == 0 && LPR <= kWave && (LPH & (LPH - 1)) == 0 && (HPW & (HPW - 1)) == 0,
                "unsupported head_dim");
  // With a 16-bit q the K products run as v_dot2 on exact 16-bit values of the codes,
  // two products per instruction with fp32 accumulation (fp32 q: one FMA per element):
  // fp8 codes by one packed conversion per two codes, in q's type; int8 codes
  // (I8F16) as the f16 numbers 1024 + (code + 128), built two at a time by one v_perm
  // from the code bytes, against q in f16 (a bf16 q multiplied by a power of two per
  // head that brings its largest element into [2^14, 2^15): exact, and undone on each
  // dot product). The K zero point then carries the 1024 + 128 offset. With one query
  // head per KV head int8 codes keep the fp32 FMAs (measured faster on MI355X for
  // MHA layers).
  constexpr bool I8F16 = DT != kF32 && QT == kI8 && GT > 1;
  constexpr bool DOT2 = DT != kF32 && (QT == kFP8 || I8F16);
  constexpr float kBias = QT == kI8 ? 128.0f : 0.0f;
  constexpr float kKBias = I8F16 ? 1152.0f : kBias;

  __shared__ uint32_t s_page[kQuantTablePages];
  // (ks, kz + K bias, vs, vz + bias) per page and head
  __shared__ float4 s_fac[kQuantTablePages][HPW];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ float s_acc[NW][GW][D];

  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = threadIdx.x / kWave;
  Partition w;
  uint32_t k0 = 0;
  if (!setup_pages<DT, D, GW, NTH, HPW>(a, grid_item<GT>(a), kKBias, kBias, s_page, s_fac, w,
                                        k0))
    return;
  const uint32_t cnt = w.cnt;
  const uint64_t out_row0 = w.out_row0;
  const uint32_t p0 = w.part * a.part_tokens;
  // a token's codes of head g start at (slot * Hkv + g) * D bytes
  const uint64_t row_bytes = uint64_t(a.num_kv_heads) * D;
  const uint64_t head0 = uint64_t(w.g) * D;

  const uint32_t row = lane / LPR;
  const uint32_t hw = (lane % LPR) / LPH;  // the lane's KV head within the workgroup's
  const uint32_t c = lane % LPH;           // the lane's chunk of that head's row

  // q of the lane's 16 elements of each head, and sum(q) over the head: packed (qw)
  // for the v_dot2 products, else fp32 (qf). qex: the exponent that undoes the
  // scaling of a bf16 q converted to f16 (I8F16).
  float qf[DOT2 ? 1 : GT][EPL], qsum[GT];
  int qex[GT];
  uint32_t qw[DOT2 ? GT : 1][EPL / 2];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const char* qp =
        static_cast<const char*>(a.q) + ((out_row0 + hw * GT + hh) * D + c * EPL) * EQ;
    float sq = 0.0f, amax = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < EPL * EQ / 16; ++h2) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * h2);
      float t[16 / EQ];
      widen16<DT>(raw, t);
#pragma unroll
      for (int e = 0; e < 16 / EQ; ++e) {
        if constexpr (DOT2) {
          sq += t[e];
          amax = fmaxf(amax, fabsf(t[e]));
        } else {
          qf[hh][h2 * (16 / EQ) + e] = t[e];
          sq += t[e];
        }
      }
      if constexpr (DOT2) {
        qw[hh][4 * h2] = raw.x;
        qw[hh][4 * h2 + 1] = raw.y;
        qw[hh][4 * h2 + 2] = raw.z;
        qw[hh][4 * h2 + 3] = raw.w;
      }
    }
    qsum[hh] = row_sum<LPH>(sq);
    qex[hh] = 0;
    if constexpr (I8F16 && DT == kBF16) {
      // the head's largest |q| over its LPH lanes sets the power of two; elements
      // under 2^-31 of it fall below f16's normal range (rounded toward zero there)
#pragma unroll
      for (int o = 1; o < LPH; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const int ex = __builtin_amdgcn_frexp_expf(amax) - 15;
      qex[hh] = ex;
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        const float lo = ldexpf(__uint_as_float(qw[hh][i] << 16), -ex);
        const float hi = ldexpf(__uint_as_float(qw[hh][i] & 0xffff0000u), -ex);
        const auto h = __builtin_amdgcn_cvt_pkrtz(lo, hi);
        __builtin_memcpy(&qw[hh][i], &h, 4);
      }
    }
  }

  float m[GT], l[GT], accz[GT], acc[GT][EPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    accz[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.0f;
  }

  const char* kbase = static_cast<const char*>(a.k_cache) + head0 + hw * D + c * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + head0 + hw * D + c * 16;

  // PF: the rows of the wave's next tile are loaded while the current one is computed
  // (kn / vn and the rows' table entries pn hold the tile in flight). Measured on
  // MI355X: int8 pools with two query heads per KV head gain (their v_dot2 K path leaves
  // the loop shorter than its loads' latency), the other shapes lose slightly and load
  // each tile at the top of its iteration instead.
  constexpr bool PF = I8F16 && GT == 2;
  // VP2: fp8 V rows taken two at a time on v_dot2_f32_bf16 (16-bit q, two query heads
  // per KV head; measured on MI355X: faster there, slower with one head per KV head)
  constexpr bool VP2 = QT == kFP8 && DT != kF32 && GT == 2 && NLOAD % 2 == 0;
  u32x4 kn[NLOAD], vn[NLOAD];
  uint32_t pn[NLOAD];
  auto load_rows = [&](uint32_t t0) {
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      const uint32_t li = t0 + k * RPL + row;
      const uint32_t p = p0 + (li < cnt ? li : cnt - 1);
      const uint32_t kp = fastdiv(p, a.page_div);
      const uint64_t slot = uint64_t(s_page[kp - k0]) * a.page_size + (p - kp * a.page_size);
      const uint64_t off = slot * row_bytes;
      kn[k] = load16<TU::NT>(kbase + off);
      vn[k] = load16<TU::NT>(vbase + off);
      pn[k] = kp - k0;
    }
  };
  if constexpr (PF) {
    if (wave * TT < cnt) load_rows(wave * TT);
  }
  for (uint32_t tb = wave * TT; tb < cnt; tb += NW * TT) {
    u32x4 kr[NLOAD], vr[NLOAD];
    float4 fac[NLOAD];
    if constexpr (PF) {
#pragma unroll
      for (int k = 0; k < NLOAD; ++k) {
        kr[k] = kn[k];
        vr[k] = vn[k];
        fac[k] = s_fac[pn[k]][hw];
      }
      if (tb + NW * TT < cnt) load_rows(tb + NW * TT);
    } else {
      // (the same loads written inline: the compiler schedules this form better here)
#pragma unroll
      for (int k = 0; k < NLOAD; ++k) {
        const uint32_t li = tb + k * RPL + row;
        const uint32_t p = p0 + (li < cnt ? li : cnt - 1);
        const uint32_t kp = fastdiv(p, a.page_div);
        const uint64_t slot = uint64_t(s_page[kp - k0]) * a.page_size + (p - kp * a.page_size);
        const uint64_t off = slot * row_bytes;
        kr[k] = load16<TU::NT>(kbase + off);
        vr[k] = load16<TU::NT>(vbase + off);
        fac[k] = s_fac[kp - k0][hw];
      }
    }

    float sc[GT][NLOAD];
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      const bool valid = tb + k * RPL + row < cnt;
      float kf[DOT2 ? 1 : EPL];
      uint32_t kw[DOT2 ? EPL / 2 : 1];
      if constexpr (I8F16) {
        // code + 128 (sign bit flipped) in the low byte of the f16 0x64xx = 1024 + byte
        const uint32_t cw[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = cw[i] ^ 0x80808080u;
          kw[2 * i] = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
          kw[2 * i + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u);
        }
      } else if constexpr (DOT2) {
        const u32x4 lo = codes8_to_bits16<DT, QT>(uint2{kr[k].x, kr[k].y});
        const u32x4 hi = codes8_to_bits16<DT, QT>(uint2{kr[k].z, kr[k].w});
        kw[0] = lo.x; kw[1] = lo.y; kw[2] = lo.z; kw[3] = lo.w;
        kw[4] = hi.x; kw[5] = hi.y; kw[6] = hi.z; kw[7] = hi.w;
      } else {
        codes16<QT>(kr[k], kf);
      }
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        float d0 = 0.0f;
        if constexpr (DOT2) {
#pragma unroll
          for (int i = 0; i < EPL / 2; ++i) {
            if constexpr (DT == kBF16 && !I8F16)
              d0 = __builtin_amdgcn_fdot2_f32_bf16(as_pair<bf16x2>(kw[i]),
                                                   as_pair<bf16x2>(qw[hh][i]), d0, false);
            else
              d0 = __builtin_amdgcn_fdot2(as_pair<f16x2>(kw[i]), as_pair<f16x2>(qw[hh][i]), d0,
                                          false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) d0 = fmaf(qf[hh][e], kf[e], d0);
        }
        float dot = row_sum<LPH>(d0);
        if constexpr (I8F16 && DT == kBF16) dot = ldexpf(dot, qex[hh]);
        const float z = fac[k].x * fmaf(-fac[k].y, qsum[hh], dot) * a.scale_log2;
        sc[hh][k] = valid ? z : -INFINITY;
      }
    }

    float mu[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float mt = sc[hh][0];
#pragma unroll
      for (int k = 1; k < NLOAD; ++k) mt = fmaxf(mt, sc[hh][k]);
      const float mn = fmaxf(m[hh], mt);
      mu[hh] = mn == -INFINITY ? 0.0f : mn;
      const float corr = __builtin_amdgcn_exp2f(m[hh] - mu[hh]);
      l[hh] *= corr;
      accz[hh] *= corr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] *= corr;
      m[hh] = mn;
    }
    if constexpr (VP2) {
      // Two rows per v_dot2: element e of rows k and k+1 as a bf16 pair (their fp8
      // codes interleaved by v_perm, then one packed conversion per two), against the
      // two rows' weights times V scale rounded to a bf16 pair. The zero-point term
      // takes the same rounded weights; the denominator sums the unrounded ones.
#pragma unroll
      for (int k = 0; k < NLOAD; k += 2) {
        const uint32_t c0[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
        const uint32_t c1[4] = {vr[k + 1].x, vr[k + 1].y, vr[k + 1].z, vr[k + 1].w};
        uint32_t vp[EPL];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = __builtin_amdgcn_perm(c1[i], c0[i], 0x05010400u);
          const uint32_t hi = __builtin_amdgcn_perm(c1[i], c0[i], 0x07030602u);
          const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
          const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
          const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
          const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
          __builtin_memcpy(&vp[4 * i], &a0, 4);
          __builtin_memcpy(&vp[4 * i + 1], &a1, 4);
          __builtin_memcpy(&vp[4 * i + 2], &a2, 4);
          __builtin_memcpy(&vp[4 * i + 3], &a3, 4);
        }
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
          const float p0 = __builtin_amdgcn_exp2f(sc[hh][k] - mu[hh]);
          const float p1 = __builtin_amdgcn_exp2f(sc[hh][k + 1] - mu[hh]);
          l[hh] += p0 + p1;
          const uint32_t wp = pack16<kBF16>(p0 * fac[k].z, p1 * fac[k + 1].z);
          accz[hh] = fmaf(__uint_as_float(wp << 16), fac[k].w, accz[hh]);
          accz[hh] = fmaf(__uint_as_float(wp & 0xffff0000u), fac[k + 1].w, accz[hh]);
          const bf16x2 w2 = as_pair<bf16x2>(wp);
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[hh][e] =
                __builtin_amdgcn_fdot2_f32_bf16(w2, as_pair<bf16x2>(vp[e]), acc[hh][e], false);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NLOAD; ++k) {
        float vf[EPL];
        codes16<QT>(vr[k], vf);
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
          const float p = __builtin_amdgcn_exp2f(sc[hh][k] - mu[hh]);
          l[hh] += p;
          const float pv = p * fac[k].z;  // weight times the token's V scale
          accz[hh] = fmaf(pv, fac[k].w, accz[hh]);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pv, vf[e], acc[hh][e]);
        }
      }
    }
  }

  // the zero-point term is common to every element of the head
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] -= accz[hh];
  }

  // Merge the RPL row groups of the wave (log-sum-exp rule).
#pragma unroll
  for (int sh = LPR; sh < kWave; sh <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float mo = __shfl_xor(m[hh], sh);
      const float lo = __shfl_xor(l[hh], sh);
      const float mn = fmaxf(m[hh], mo);
      const float mref = mn == -INFINITY ? 0.0f : mn;
      const float fa = __builtin_amdgcn_exp2f(m[hh] - mref);
      const float fb = __builtin_amdgcn_exp2f(mo - mref);
      l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[hh][e], sh);
        acc[hh][e] = acc[hh][e] * fa + ao * fb;
      }
      m[hh] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][hw * GT + hh][c * EPL + e] = acc[hh][e];
      if (c == 0) {
        s_m[wave][hw * GT + hh] = m[hh];
        s_l[wave][hw * GT + hh] = l[hh];
      }
    }
  }
  __syncthreads();

  finish_partition<DT, D, GW, NW>(a, w, s_m, s_l, s_acc);
}

// ---------------------------------------------------------------------------
// GQA groups of 4 or more query heads: q.K^T and P.V on the matrix cores.
//
// Per wave and 32-token tile (two 16-token groups), with v_mfma_f32_16x16x32
// (bf16 or f16 inputs, fp32 accumulate; lane layout: A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16], D[4(l/16)+r][l%16]):
//   * K and V rows are loaded row-major (16-byte lane loads, whole rows per
//     group of lanes, the pattern that streams at the HBM ceiling) and
//     written to this wave's LDS tile, rows padded by 16 bytes so the operand
//     reads below hit distinct banks;
//   * scores: S^T[token][head] = K Q^T, A = K read back per token row, B = q
//     (columns are the tile's query heads, unused columns zero). Lane l ends
//     with tokens 16g+4(l/16)+r of head l%16;
//   * online softmax per head in base 2; the running max is shared by the four
//     lanes holding the head (shuffles across lane quarters);
//   * P.V: O^T[d][head] = V^T P^T. The contraction index k = 8(l/16)+j is
//     mapped to token 16(j/4)+4(l/16)+(j%4), which is exactly where the scores
//     already sit, so P needs no data movement; V^T is gathered from LDS in
//     the same token order (by the transposing LDS read below, from V rows
//     padded by 32 bytes). P is rounded to the input type for the matrix
//     cores and the softmax denominator sums the rounded weights.
// The next tile's loads are issued before the current tile is computed.
// ---------------------------------------------------------------------------

// Max over the four lanes l, l^16, l^32, l^48 that hold one column of a
// 16x16 MFMA result (v_permlane32_swap / v_permlane16_swap exchange whole 32-
// and 16-lane halves, without the LDS round trip of a shuffle), as IEEE
// maximum: gfx950's v_maximum, which needs no quieting instructions. A NaN
// score makes its head's result NaN under either maximum.
__device__ inline float col_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ds_read_b64_tr_b16 (gfx950 transposing LDS read): within each group of 16
// lanes, lanes 4r..4r+3 fetch the 16 elements of row r of a 4x16 block (8 bytes
// each) and lane i receives column i of the four rows. Returns this lane's four
// 16-bit results packed in two words; p must be 8-byte aligned.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ inline uint2 lds_read_tr16(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((lds_char*)(const_cast<char*>(p))));
  uint2 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

template <int DT, int D, int GT, int HPW, int SPLIT, int MINW, int CB = 1>
__global__ __launch_bounds__(HPW * SPLIT * 64, MINW) void decode_partition_mfma_kernel(
    const DecodeKernelArgs a) {
  static_assert(DT != kF32 && D % 32 == 0 && D <= 128 && GT <= 16, "unsupported shape");
  constexpr int NW = HPW * SPLIT;  // waves: HPW adjacent KV heads, SPLIT waves per head
  constexpr int NTH = NW * kWave;
  constexpr int CPR = D / 8;       // 16-byte chunks per token row
  constexpr int LPR = CPR;         // lanes per row in the row-major loads
  constexpr int RPL = kWave / LPR; // rows per wave load
  constexpr int TT = 32;           // tokens per tile
  constexpr int NL = TT / RPL;     // wave loads per tile, for K and for V
  constexpr int KROW = D * 2 + 16; // LDS bytes per K row (16-byte lane reads: distinct banks)
  constexpr int VROW = D * 2 + 32; // LDS bytes per V row (transposing 8-byte reads likewise)
  constexpr int KS = D / 32;       // score MFMAs per 16 tokens (d steps)
  constexpr int NB = D / 16;       // P.V MFMAs per tile (16-column blocks of d)
  // A shared run fills CB blocks of 16 tile columns (CB = 1 on the plain decode): each
  // K and V operand read from LDS feeds CB matrix-core products.
  constexpr int R = CB * 16 / GT;  // sequences a shared run can bring into the columns
  constexpr int NC = R * GT;       // columns in use when a run fills them (16 * CB)

  // two-head workgroups: pool slots (32 bits) for up to kLongPartTokens tokens, so
  // the table stays at 8 KB and two workgroups still share a CU; else offsets
  using RowT = std::conditional_t<(HPW > 1), uint32_t, uint64_t>;
  __shared__ RowT s_row[HPW > 1 ? kLongPartTokens : kMaxPartTokens];
  __shared__ __attribute__((aligned(16))) char s_tile[NW][TT * (KROW + VROW)];
  __shared__ float s_m[NW][NC];
  __shared__ float s_l[NW][NC];
  __shared__ uint32_t s_np[R];  // partitions of each served sequence
  static_assert(sizeof(float) * NC * D <= TT * (KROW + VROW), "merge buffer must fit the tiles");

  const uint32_t lane = threadIdx.x % kWave;
  // wave-uniform: kept in a scalar register, so the tile loop branches are scalar
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t hw = wave % HPW;   // the wave's KV head within the workgroup's heads
  const uint32_t sub = wave / HPW;  // the wave's share of the partition's tiles
  Partition w;
  const WorkItem item = grid_item<GT, (HPW > 1)>(a);
  // s_row holds the rows of the first KV head; head hw's rows follow at hw*D
  if (!setup_partition<DT, D, HPW * GT, NTH, NoTokenHook, HPW>(a, item, s_row, w)) return;
  const uint32_t cnt = w.cnt;

  // A shared run: sequences s .. s+members-1 read exactly these rows for this
  // partition (the ordering pass checked every page id), so each gets GT columns of
  // the tile; a column of a matrix-core result depends only on its own q column,
  // so every member gets the arithmetic of its own workgroup.
  const uint32_t members = R > 1 ? min(item.members, uint32_t(R)) : 1u;
  if (threadIdx.x < members)
    s_np[threadIdx.x] =
        threadIdx.x == 0 ? w.nparts : num_parts(a.context_lens[w.s + threadIdx.x], a.part_tokens);
  const uint32_t ncol = members * GT;  // columns in use: member c / GT, head c % GT

  const uint32_t q4 = lane / 16;   // lane quarter
  const uint32_t col = lane % 16;  // MFMA column; column c = 16 * cb + col of block cb

  u32x4 qop[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const uint32_t c = 16 * cb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[cb][ks] = u32x4{0, 0, 0, 0};
      if (c < ncol) {
        const uint64_t row = w.out_row0 + uint64_t(c / GT) * a.num_q_heads + hw * GT + c % GT;
        const char* qp = static_cast<const char*>(a.q) + (row * D + 32 * ks + 8 * q4) * 2;
        qop[cb][ks] = *reinterpret_cast<const u32x4*>(qp);
      }
    }
  }

  f32x4 acc[CB][NB];
  float m[CB], l[CB];  // running max (base 2) and weight sum of column 16 * cb + col
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = -INFINITY;
    l[cb] = 0.0f;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[cb][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const uint32_t lr = lane / LPR, lc = lane % LPR;  // row-major load: row, 16-byte chunk
  char* kt = s_tile[wave];
  char* vt = s_tile[wave] + TT * KROW;
  // with a slot table, head g's row of a token starts g*D elements into its pool row
  const uint64_t row_bytes = uint64_t(a.num_kv_heads) * D * 2;
  const uint64_t head0 = HPW > 1 ? uint64_t(w.g) * D : 0;
  const char* kbase = static_cast<const char*>(a.k_cache) + (head0 + hw * D + lc * 8) * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (head0 + hw * D + lc * 8) * 2;

  uint32_t tb = sub * TT;
  if (tb < cnt) {
    u32x4 kr[NL], vr[NL];
    auto load_tile = [&](uint32_t t0) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t li = t0 + i * RPL + lr;
        const uint64_t off = HPW > 1 ? uint64_t(s_row[li < cnt ? li : cnt - 1]) * row_bytes
                                     : uint64_t(s_row[li < cnt ? li : cnt - 1]) * 2;
        kr[i] = load16<true>(kbase + off);
        vr[i] = load16<true>(vbase + off);
      }
    };
    auto store_tile = [&]() {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t r = i * RPL + lr;
        *reinterpret_cast<u32x4*>(kt + r * KROW + lc * 16) = kr[i];
        *reinterpret_cast<u32x4*>(vt + r * VROW + lc * 16) = vr[i];
      }
    };
    load_tile(tb);
    store_tile();
    while (true) {
      const uint32_t tn = tb + SPLIT * TT;
      const bool has_next = tn < cnt;
      if (has_next) load_tile(tn);

      // scores of tokens 16g + 4*q4 + r for column `col` of each block
      f32x4 sacc[CB][2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) sacc[cb][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kop =
              *reinterpret_cast<const u32x4*>(kt + (16 * g + col) * KROW + (32 * ks + 8 * q4) * 2);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            sacc[cb][g] = mfma_16x16x32<DT>(kop, qop[cb][ks], sacc[cb][g]);
        }
      }
      u32x4 pop[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t t = 16 * (j / 4) + 4 * q4 + (j % 4);
          const float zz = sacc[cb][j / 4][j % 4] * a.scale_log2;
          z[j] = tb + t < cnt ? zz : -INFINITY;
        }
        float mt = z[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, z[j]);
        mt = col_max4(mt);
        const float mn = fmaxf(m[cb], mt);
        const float mu = mn == -INFINITY ? 0.0f : mn;
        const float corr = __builtin_amdgcn_exp2f(m[cb] - mu);
        m[cb] = mn;
        l[cb] *= corr;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[cb][n] *= corr;

        uint32_t pw[4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const uint32_t b = pack16<DT>(__builtin_amdgcn_exp2f(z[j] - mu),
                                        __builtin_amdgcn_exp2f(z[j + 1] - mu));
          psum += widen_bits16<DT>(b & 0xffffu) + widen_bits16<DT>(b >> 16);
          pw[j / 2] = b;
        }
        // Columns c >= ncol carry q = 0: scores 0 (or -inf past the context), finite
        // weights. A column of an MFMA result depends only on the same column of its B
        // operand, so they never reach a served head, and they are never stored.
        l[cb] += psum;
        pop[cb] = u32x4{pw[0], pw[1], pw[2], pw[3]};
      }

      // V^T: lane (q4, col) fetches row 4*q4 + col/4 (and 16 + that), columns
      // 16n + 4*(col%4) .. +3, and receives column 16n + col
      const char* vrow0 = vt + (4 * q4 + col / 4) * VROW + 8 * (col % 4);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const uint2 lo = lds_read_tr16(vrow0 + 32 * n);
        const uint2 hi = lds_read_tr16(vrow0 + 16 * VROW + 32 * n);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][n] = mfma_16x16x32<DT>(u32x4{lo.x, lo.y, hi.x, hi.y}, pop[cb], acc[cb][n]);
      }
      if (!has_next) break;
      store_tile();
      tb = tn;
    }
  }

  __syncthreads();  // every wave is done with its tile before the tiles become merge space
  float(*s_acc)[NC][D] = reinterpret_cast<float(*)[NC][D]>(&s_tile[0][0]);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    // the four lane quarters hold disjoint tokens of each column: add their sums
    float ls = l[cb];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    const uint32_t c = 16 * cb + col;
    if (c < ncol) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s_acc[wave][c][16 * n + 4 * q4 + r] = acc[cb][n][r];
      }
      if (q4 == 0) {
        s_m[wave][c] = m[cb];
        s_l[wave][c] = ls;
      }
    }
  }
  __syncthreads();
  // Merge the waves of each served column (log-sum-exp rule) and write the result, or
  // the partition's partial when the column's sequence has several partitions: the
  // arithmetic of finish_partition, per served sequence.
  for (uint32_t i = threadIdx.x; i < HPW * ncol * D; i += NTH) {
    const uint32_t hw_ = i / (ncol * D), c = (i / D) % ncol, e = i % D;
    float mx = s_m[hw_][c];
#pragma unroll
    for (int v = 1; v < SPLIT; ++v) mx = fmaxf(mx, s_m[v * HPW + hw_][c]);
    const float mref = mx == -INFINITY ? 0.0f : mx;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int v = 0; v < SPLIT; ++v) {
      const float f = __builtin_amdgcn_exp2f(s_m[v * HPW + hw_][c] - mref);
      L = fmaf(s_l[v * HPW + hw_][c], f, L);
      O = fmaf(s_acc[v * HPW + hw_][c][e], f, O);
    }
    const uint64_t row = w.out_row0 + uint64_t(c / GT) * a.num_q_heads + hw_ * GT + c % GT;
    if (s_np[c / GT] == 1) {
      store_out<DT>(a.out, row * D + e, L > 0.0f ? O / L : 0.0f);
    } else {
      const uint64_t r = row * a.max_parts + w.part;
      a.ws_o[r * D + e] = O;
      if (e == 0) a.ws_ml[r] = make_float2(mx, L);
    }
  }
}

// ---------------------------------------------------------------------------
// Quantized pools, GQA groups of 4 or more query heads, 16-bit q: the matrix-
// core kernel above on one-byte codes. Each lane loads 16 codes of a row
// (half the bytes per token of a 16-bit pool). V codes go to the wave's LDS tile
// as exact 16-bit values (int8 codes as code + 128 in 0..255, E4M3 values; both
// exact in bf16 and in f16); K stays one byte per code in LDS, and each lane
// converts the 8 codes of its operand as it reads them. Every code is converted
// once either way, and the smaller tile lets four workgroups share a CU instead
// of three. The two products are those of the 16-bit kernel over raw code
// values; the page factors of token t enter around them:
//   score = ks_t * (q . value_t - kz_t * sum(q)),   weight' = p_t * vs_t,
//   out   = (sum_t weight'_t value_t - sum_t weight'_t vz_t) / sum_t p_t,
// with the bias of int8 codes folded into the zero points. V^T is read with the
// transposing LDS read ds_read_b64_tr_b16 (lanes 4r..4r+3 of each 16-lane group
// fetch row r of a 4x16 block; lane i receives column i), from rows padded by
// 32 bytes so those 8-byte reads fall on distinct banks.
// ---------------------------------------------------------------------------

template <int DT, int QT, int D, int GT, class TU, int HPW>
__global__ __launch_bounds__(TU::NW * 64, TU::MINW) void decode_partition_mfma_quant_kernel(
    const DecodeKernelArgs a) {
  static_assert(DT != kF32 && D % 32 == 0 && D <= 128 && GT <= 16, "unsupported shape");
  constexpr int NW = TU::NW;          // HPW adjacent KV heads, NW / HPW waves per head
  constexpr int SPLIT = NW / HPW;
  static_assert(NW % HPW == 0, "waves per head");
  constexpr int NTH = NW * kWave;
  constexpr int LPR = D / 16;       // lanes per row: 16 codes per lane
  constexpr int RPL = kWave / LPR;  // rows per wave load
  constexpr int TT = 32;            // tokens per tile
  constexpr int NL = TT / RPL;      // wave loads per tile, for K and for V
  constexpr int KROW = D + 16;      // LDS bytes per K row of codes (8-byte lane reads)
  constexpr int VROW = D * 2 + 32;  // LDS bytes per V row (transposing 8-byte reads)
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr float kBias = QT == kI8 ? 128.0f : 0.0f;

  __shared__ uint32_t s_page[kQuantTablePages];
  __shared__ float4 s_fac[kQuantTablePages][HPW];  // (ks, kz + bias, vs, vz + bias) per page, head
  __shared__ __attribute__((aligned(16))) char s_tile[NW][TT * (KROW + VROW)];
  __shared__ float s_m[NW][GT];
  __shared__ float s_l[NW][GT];
  static_assert(sizeof(float) * GT * D <= TT * (KROW + VROW), "merge buffer must fit the tiles");

  const uint32_t lane = threadIdx.x % kWave;
  // wave-uniform: kept in a scalar register, so the tile loop branches are scalar
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t hw = wave % HPW;   // the wave's KV head within the workgroup's heads
  const uint32_t sub = wave / HPW;  // the wave's share of the partition's tiles
  Partition w;
  uint32_t k0 = 0;
  if (!setup_pages<DT, D, HPW * GT, NTH, HPW>(a, grid_item<GT, (HPW > 1)>(a), kBias, kBias, s_page,
                                              s_fac, w, k0))
    return;
  const uint32_t cnt = w.cnt;

  const uint32_t q4 = lane / 16;
  const uint32_t col = lane % 16;
  const bool pg4 = a.page_size % 4 == 0;

  // Scores are kept raw, ks * (q.value - kz * sum(q)), and scaled by
  // c = |scale| * log2(e) inside the exponent; a negative scale is a sign flip of q
  // (exact, and it flips sum(q) with it). Lazy rescaling: the subtracted max is
  // raised only when a head's max grows by more than 8 (log2 units), so weights stay
  // below 2^8 and most tiles skip the rescale of the accumulators.
  const float c = fmaxf(fabsf(a.scale_log2), FLT_MIN);  // > 0 (a zero scale acts as FLT_MIN)
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  const float thr = 8.0f / c;
  u32x4 qop[KS];
  float qpart = 0.0f;  // this lane's share of sum(q) of head `col`
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = u32x4{0, 0, 0, 0};
    if (col < GT) {
      const char* qp =
          static_cast<const char*>(a.q) + ((w.out_row0 + hw * GT + col) * D + 32 * ks + 8 * q4) * 2;
      qop[ks] = *reinterpret_cast<const u32x4*>(qp) ^ qflip;
      float f[8];
      widen16<DT>(qop[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qpart += f[e];
    }
  }
  qpart += __shfl_xor(qpart, 16);
  const float qsum = qpart + __shfl_xor(qpart, 32);

  f32x4 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float l = 0.0f, accz = 0.0f;
  float mthr = -INFINITY, mc = 0.0f;  // rescale threshold (raw units), subtracted max * c

  const uint32_t lr = lane / LPR, lc = lane % LPR;  // row-major load: row, 16-code chunk
  char* kt = s_tile[wave];
  char* vt = s_tile[wave] + TT * KROW;
  // a token's codes of head g start at (slot * Hkv + g) * D bytes
  const uint32_t p0 = w.part * a.part_tokens;
  const uint64_t row_bytes = uint64_t(a.num_kv_heads) * D;
  const char* kbase = static_cast<const char*>(a.k_cache) + (uint64_t(w.g) + hw) * D + lc * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + (uint64_t(w.g) + hw) * D + lc * 16;

  uint32_t tb = sub * TT;
  if (tb < cnt) {
    u32x4 kr[NL], vr[NL];
    // rows past the partition (only in its last tile) reuse its last row
    auto load_tile = [&](auto full_tag, uint32_t t0) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t li = t0 + i * RPL + lr;
        const uint32_t p = p0 + (FULL || li < cnt ? li : cnt - 1);
        const uint32_t kp = fastdiv(p, a.page_div);
        const uint64_t off =
            (uint64_t(s_page[kp - k0]) * a.page_size + (p - kp * a.page_size)) * row_bytes;
        kr[i] = load16<TU::NT>(kbase + off);
        vr[i] = load16<TU::NT>(vbase + off);
      }
    };
    auto store_tile = [&]() {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t r = i * RPL + lr;
        *reinterpret_cast<u32x4*>(kt + r * KROW + lc * 16) = kr[i];  // K stays codes
        u32x4 lo, hi;
        codes16_to_bits16<DT, QT>(vr[i], lo, hi);
        *reinterpret_cast<u32x4*>(vt + r * VROW + lc * 32) = lo;
        *reinterpret_cast<u32x4*>(vt + r * VROW + lc * 32 + 16) = hi;
      }
    };
    // scores, online softmax and P.V of the tile at tb; FULL: every token is in the
    // partition, so no score needs masking
    auto compute_tile = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      f32x4 sacc[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        sacc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint2 kc =
              *reinterpret_cast<const uint2*>(kt + (16 * g + col) * KROW + 32 * ks + 8 * q4);
          sacc[g] = mfma_16x16x32<DT>(codes8_to_bits16<DT, QT>(kc), qop[ks], sacc[g]);
        }
      }
      float sv[8];
      float4 fac[8];
      if (pg4) {
        // the lane's tokens 4*q4 .. +3 of each 16-token group start at a multiple of 4
        // (partitions and tiles do), so they share one page
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t t = tb + 16 * h + 4 * q4;
          const float4 f = s_fac[fastdiv(p0 + (FULL ? t : min(t, cnt - 1)), a.page_div) - k0][hw];
#pragma unroll
          for (int r = 0; r < 4; ++r) fac[4 * h + r] = f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t t = tb + 16 * (j / 4) + 4 * q4 + (j % 4);
          fac[j] = s_fac[fastdiv(p0 + (FULL || t < cnt ? t : cnt - 1), a.page_div) - k0][hw];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sv[j] = fac[j].x * fmaf(-fac[j].y, qsum, sacc[j / 4][j % 4]);
        if constexpr (!FULL) {
          if (tb + 16 * (j / 4) + 4 * q4 + (j % 4) >= cnt) sv[j] = -INFINITY;
        }
      }
      float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mt = col_max4(mt);
      const bool need = mt > mthr;
      if (__any(need)) {
        const float mcn = need ? mt * c : mc;
        // no earlier weights on first use (mthr still -inf): the accumulators are zero
        const float corr = mthr == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc - mcn);
        if (need) mthr = mt + thr;
        mc = mcn;
        l *= corr;
        accz *= corr;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] *= corr;
      }
      // masked scores are -inf and c > 0, so their weight is exactly 0. Columns
      // col >= GT carry q = 0 and finite weights; a column of an MFMA result depends
      // only on the same column of its B operand, so they never reach a served head.
      uint32_t pw[4];
      float psum = 0.0f, zsum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[j], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[j + 1], c, -mc));
        const uint32_t b = pack16<DT>(p0 * fac[j].z, p1 * fac[j + 1].z);
        psum += p0 + p1;
        zsum = fmaf(widen_bits16<DT>(b & 0xffffu), fac[j].w, zsum);
        zsum = fmaf(widen_bits16<DT>(b >> 16), fac[j + 1].w, zsum);
        pw[j / 2] = b;
      }
      l += psum;
      accz += zsum;
      const u32x4 pop = u32x4{pw[0], pw[1], pw[2], pw[3]};

      // V^T: lane (q4, col) fetches row 4*q4 + col/4 (and 16 + that), columns
      // 16n + 4*(col%4) .. +3, and receives column 16n + col
      const char* vrow0 = vt + (4 * q4 + col / 4) * VROW + 8 * (col % 4);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const uint2 lo = lds_read_tr16(vrow0 + 32 * n);
        const uint2 hi = lds_read_tr16(vrow0 + 16 * VROW + 32 * n);
        acc[n] = mfma_16x16x32<DT>(u32x4{lo.x, lo.y, hi.x, hi.y}, pop, acc[n]);
      }
    };
    if (tb + TT <= cnt) load_tile(std::true_type{}, tb);
    else load_tile(std::false_type{}, tb);
    store_tile();
    while (true) {
      const uint32_t tn = tb + SPLIT * TT;
      const bool has_next = tn < cnt;
      if (has_next) {
        if (tn + TT <= cnt) load_tile(std::true_type{}, tn);
        else load_tile(std::false_type{}, tn);
      }
      if (tb + TT <= cnt) compute_tile(std::true_type{});
      else compute_tile(std::false_type{});
      if (!has_next) break;
      store_tile();
      tb = tn;
    }
  }

  // the four lane quarters hold disjoint tokens of each head: add their sums
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  accz += __shfl_xor(accz, 16);
  accz += __shfl_xor(accz, 32);
  __syncthreads();  // every wave is done with its tile before the tiles become merge space
  float(*s_acc)[GT][D] = reinterpret_cast<float(*)[GT][D]>(&s_tile[0][0]);
  if (col < GT) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_acc[wave][col][16 * n + 4 * q4 + r] = acc[n][r] - accz;
    }
    if (q4 == 0) {  // a wave that saw no token of the head reports max -inf and sum 0
      s_m[wave][col] = mthr == -INFINITY ? -INFINITY : mc;
      s_l[wave][col] = l;
    }
  }
  __syncthreads();
  finish_partition<DT, D, GT, NW, HPW>(a, w, s_m, s_l, s_acc);
}

// One wave per (sequence, query head) with more than one partition: merges the
// partitions with the log-sum-exp rule, normalises and rounds to dtype. Lane j
// reads partition j's (max, sum) so the partials are fetched in parallel; the
// weights are then shared through the wave's lanes.
template <int DT>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(const ReduceKernelArgs a) {
  const uint32_t lane = threadIdx.x % kWave;
  const uint64_t sh = uint64_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
  if (sh >= uint64_t(a.num_seqs) * a.num_q_heads) return;
  const uint32_t s = uint32_t(sh / a.num_q_heads);
  const int32_t n = a.context_lens[s];
  if (length_is_bad(n, a.max_context_len)) return;
  const uint32_t nparts = num_parts(n, a.part_tokens);
  if (nparts <= 1) return;
  const float2* ml = a.ws_ml + sh * a.max_parts;
  const float* o = a.ws_o + sh * a.max_parts * a.head_dim;
  // global max over partitions: lane j holds partition j, j + 64, ...
  float mx = -INFINITY;
  for (uint32_t j = lane; j < nparts; j += kWave) mx = fmaxf(mx, ml[j].x);
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sft));
  // weight of partition `lane` (the first 64 partitions), and the total weight
  float wl = 0.0f, L = 0.0f;
  for (uint32_t j = lane; j < nparts; j += kWave) {
    const float2 v = ml[j];
    const float f = __builtin_amdgcn_exp2f(v.x - mx);
    if (j == lane) wl = f;
    L = fmaf(v.y, f, L);
  }
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) L += __shfl_xor(L, sft);
  // weighted sum of the partial vectors, partitions in order; every lane runs
  // every iteration (the weights are read from lane j with v_readlane)
  for (uint32_t e0 = 0; e0 < a.head_dim; e0 += kWave) {
    const uint32_t e = e0 + lane;
    const bool active = e < a.head_dim;
    float O = 0.0f;
#pragma unroll 8
    for (uint32_t j = 0; j < nparts; ++j) {
      const float f = j < uint32_t(kWave)
                          ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), int(j)))
                          : __builtin_amdgcn_exp2f(ml[j].x - mx);
      const float v = active ? o[uint64_t(j) * a.head_dim + e] : 0.0f;
      O = fmaf(v, f, O);
    }
    if (active) store_out<DT>(a.out, sh * a.head_dim + e, O / L);
  }
}

// Launch shapes measured on MI355X (bf16, d=128): for one query head per KV
// head the kernel streams at the HBM ceiling with 8-wave workgroups and 8 row
// loads per lane in flight; wider GQA tiles are VALU-heavy and run best with
// fewer loads per tile and the register budget capped for 4 waves per SIMD.
template <int DT, int D, int GT>
struct DefaultTune {
  using type = Tune<GT == 1 ? 8 : 4, GT == 1 ? 8 : 4, true, GT >= 8 ? 2 : 4>;
};

template <int DT, int D, int GT>
hipError_t launch_pd(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  using TU = typename DefaultTune<DT, D, GT>::type;
  switch (a.kv_per_wg) {
    case 1:
      hipLaunchKernelGGL((decode_partition_kernel<DT, D, GT, TU, 1>), dim3(uint32_t(nwg)),
                         dim3(TU::NW * kWave), 0, stream, a);
      break;
    case 2:
      if constexpr (2 * D * Elem<DT>::bytes <= 16 * kWave) {
        hipLaunchKernelGGL((decode_partition_kernel<DT, D, GT, TU, 2>), dim3(uint32_t(nwg)),
                           dim3(TU::NW * kWave), 0, stream, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    case 4:
      if constexpr (4 * D * Elem<DT>::bytes <= 16 * kWave) {
        hipLaunchKernelGGL((decode_partition_kernel<DT, D, GT, TU, 4>), dim3(uint32_t(nwg)),
                           dim3(TU::NW * kWave), 0, stream, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Matrix-core path: 16-bit inputs, head_dim a multiple of 32 up to 128, and
// at least 4 query heads per KV head (below that the VALU kernel already
// streams at the bandwidth ceiling).
inline bool mfma_eligible(int dtype, uint32_t head_dim, uint32_t group) {
  return dtype != kF32 && (head_dim == 32 || head_dim == 64 || head_dim == 128) &&
         group % 4 == 0;
}

template <int DT, int D, int GT, int HPW, int SPLIT>
hipError_t launch_pm_shape(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  // shared runs longer than one block of 16 columns take two blocks
  if constexpr (GT <= 8) {
    if (a.share_block > 16 / GT) {
      hipLaunchKernelGGL((decode_partition_mfma_kernel<DT, D, GT, HPW, SPLIT, 2, 2>),
                         dim3(uint32_t(nwg)), dim3(HPW * SPLIT * kWave), 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_partition_mfma_kernel<DT, D, GT, HPW, SPLIT, 2>), dim3(uint32_t(nwg)),
                     dim3(HPW * SPLIT * kWave), 0, stream, a);
  return hipGetLastError();
}

// Two waves share each KV head's tiles. A workgroup serves one KV head, or two
// adjacent ones when a tile holds the whole GQA group: it then reads 2*d*b
// contiguous bytes of each token row and covers 1024- or 2048-token partitions, so its
// fixed costs (row table, first loads, merge) are spread over four times the
// bytes. Measured on MI355X (bf16, d=128, GQA 32/8): 5.2 -> 5.6 TB/s on mixed
// lengths, 5.6 -> 6.3 TB/s on equal ones.
template <int DT, int D, int GT>
hipError_t launch_pm(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  switch (a.kv_per_wg) {
    case 1: return launch_pm_shape<DT, D, GT, 1, 2>(a, nwg, stream);
    case 2: return launch_pm_shape<DT, D, GT, 2, 2>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_d(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  const uint32_t gt = heads_per_workgroup(DT, D, a.group);
  if constexpr (DT != kF32 && D >= 32 && D <= 128) {
    if (mfma_eligible(DT, D, a.group)) {
      switch (gt) {
        case 4: return launch_pm<DT, D, 4>(a, nwg, stream);
        case 8: return launch_pm<DT, D, 8>(a, nwg, stream);
        case 16: return launch_pm<DT, D, 16>(a, nwg, stream);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (gt) {
    case 1: return launch_pd<DT, D, 1>(a, nwg, stream);
    case 2: return launch_pd<DT, D, 2>(a, nwg, stream);
    case 4: return launch_pd<DT, D, 4>(a, nwg, stream);
    case 8: return launch_pd<DT, D, 8>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_dt(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                     hipStream_t stream) {
  switch (head_dim) {
    case 8: return launch_d<DT, 8>(a, nwg, stream);
    case 16: return launch_d<DT, 16>(a, nwg, stream);
    case 32: return launch_d<DT, 32>(a, nwg, stream);
    case 64: return launch_d<DT, 64>(a, nwg, stream);
    case 128: return launch_d<DT, 128>(a, nwg, stream);
    case 256: return launch_d<DT, 256>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int QT, int D, int GT>
hipError_t launch_quant(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  // Two-wave workgroups keep the most waves resident (the loop is latency-bound:
  // converting and FMA-ing one-byte codes leaves no loads in flight for long);
  // 4-head tiles hold 64 q floats per lane, so they load two rows per lane. Two
  // adjacent KV heads per workgroup read 2*d contiguous bytes of each token row:
  // rows of one 128-byte line per head stream markedly slower on MI355X.
  // (int8 codes with a 16-bit q and two heads per tile: 4 rows, prefetched a tile ahead)
  using TU = Tune<2, GT >= 4 ? 2 : (DT != kF32 && QT == kI8 && GT == 2 ? 4 : 8), true, 2>;
  switch (a.kv_per_wg) {
    case 1:
      hipLaunchKernelGGL((decode_partition_quant_kernel<DT, QT, D, GT, TU, 1>),
                         dim3(uint32_t(nwg)), dim3(TU::NW * kWave), 0, stream, a);
      break;
    case 2:
      hipLaunchKernelGGL((decode_partition_quant_kernel<DT, QT, D, GT, TU, 2>),
                         dim3(uint32_t(nwg)), dim3(TU::NW * kWave), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT, int QT, int D, int GT>
hipError_t launch_quant_mfma(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  // two waves per KV head; one KV head per workgroup, or two adjacent ones (whole GQA
  // groups) whose codes are 2*d contiguous bytes of each token row
  switch (a.kv_per_wg) {
    case 1: {
      using TU = Tune<2, 0, true, 2>;
      hipLaunchKernelGGL((decode_partition_mfma_quant_kernel<DT, QT, D, GT, TU, 1>),
                         dim3(uint32_t(nwg)), dim3(TU::NW * kWave), 0, stream, a);
      break;
    }
    case 2: {
      using TU = Tune<4, 0, true, 2>;
      hipLaunchKernelGGL((decode_partition_mfma_quant_kernel<DT, QT, D, GT, TU, 2>),
                         dim3(uint32_t(nwg)), dim3(TU::NW * kWave), 0, stream, a);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

inline bool mfma_quant_eligible(int dtype, uint32_t head_dim, uint32_t group) {
  return dtype != kF32 && (head_dim == 32 || head_dim == 64 || head_dim == 128) &&
         group % 4 == 0;
}

template <int DT, int QT, int D>
hipError_t launch_quant_d(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  if constexpr (DT != kF32 && D >= 32 && D <= 128) {
    if (mfma_quant_eligible(DT, D, a.group)) {
      switch (heads_per_workgroup_quant(DT, D, a.group)) {
        case 4: return launch_quant_mfma<DT, QT, D, 4>(a, nwg, stream);
        case 8: return launch_quant_mfma<DT, QT, D, 8>(a, nwg, stream);
        case 16: return launch_quant_mfma<DT, QT, D, 16>(a, nwg, stream);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (heads_per_workgroup_quant(DT, D, a.group)) {
    case 1: return launch_quant<DT, QT, D, 1>(a, nwg, stream);
    case 2: return launch_quant<DT, QT, D, 2>(a, nwg, stream);
    case 4: return launch_quant<DT, QT, D, 4>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int QT>
hipError_t launch_quant_dt(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                           hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_quant_d<DT, QT, 16>(a, nwg, stream);
    case 32: return launch_quant_d<DT, QT, 32>(a, nwg, stream);
    case 64: return launch_quant_d<DT, QT, 64>(a, nwg, stream);
    case 128: return launch_quant_d<DT, QT, 128>(a, nwg, stream);
    case 256: return launch_quant_d<DT, QT, 256>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_quant_kv(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                           uint64_t nwg, hipStream_t stream) {
  switch (kv_type) {
    case kI8: return launch_quant_dt<DT, kI8>(head_dim, a, nwg, stream);
    case kFP8: return launch_quant_dt<DT, kFP8>(head_dim, a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

#if HPKV_DECODE_HAS(1)
hipError_t launch_decode_f32(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                             hipStream_t stream) {
  return launch_dt<kF32>(head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(2)
hipError_t launch_decode_f16(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                             hipStream_t stream) {
  return launch_dt<kF16>(head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(3)
hipError_t launch_decode_bf16(uint32_t head_dim, const DecodeKernelArgs& a, uint64_t nwg,
                              hipStream_t stream) {
  return launch_dt<kBF16>(head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(4)
hipError_t launch_decode_quant_f32(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                   uint64_t nwg, hipStream_t stream) {
  return launch_quant_kv<kF32>(kv_type, head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(5)
hipError_t launch_decode_quant_f16(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                   uint64_t nwg, hipStream_t stream) {
  return launch_quant_kv<kF16>(kv_type, head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(6)
hipError_t launch_decode_quant_bf16(int kv_type, uint32_t head_dim, const DecodeKernelArgs& a,
                                    uint64_t nwg, hipStream_t stream) {
  return launch_quant_kv<kBF16>(kv_type, head_dim, a, nwg, stream);
}
#endif

#if HPKV_DECODE_HAS(0)
uint32_t heads_per_workgroup_quant(int dtype, uint32_t head_dim, uint32_t group) {
  if (mfma_quant_eligible(dtype, head_dim, group))
    return group % 16 == 0 ? 16 : group % 8 == 0 ? 8 : 4;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

hipError_t launch_decode_partitions_quant(int dtype, int kv_type, uint32_t head_dim,
                                          const DecodeKernelArgs& a, uint64_t num_workgroups,
                                          hipStream_t stream) {
  const hipError_t e = launch_order(a, stream);
  if (e != hipSuccess) return e;
  switch (dtype) {
    case kF32: return launch_decode_quant_f32(kv_type, head_dim, a, num_workgroups, stream);
    case kF16: return launch_decode_quant_f16(kv_type, head_dim, a, num_workgroups, stream);
    case kBF16: return launch_decode_quant_bf16(kv_type, head_dim, a, num_workgroups, stream);
    default: return hipErrorInvalidValue;
  }
}

uint32_t heads_per_workgroup(int dtype, uint32_t head_dim, uint32_t group) {
  if (mfma_eligible(dtype, head_dim, group)) return group % 16 == 0 ? 16 : group % 8 == 0 ? 8 : 4;
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

bool decode_on_matrix_cores(int dtype, uint32_t head_dim, uint32_t group) {
  return mfma_eligible(dtype, head_dim, group);
}

bool decode_quant_on_matrix_cores(int dtype, uint32_t head_dim, uint32_t group) {
  return mfma_quant_eligible(dtype, head_dim, group);
}

uint32_t kv_heads_per_workgroup(int dtype, uint32_t head_dim, uint32_t group,
                                uint32_t num_kv_heads) {
  if (heads_per_workgroup(dtype, head_dim, group) != group || num_kv_heads % 2 != 0) return 1;
  if (mfma_eligible(dtype, head_dim, group)) return 2;
  // VALU kernel: heads until a token's row for the workgroup is ~512 contiguous
  // bytes (measured on MI355X: 256-byte head rows stream best two at a time,
  // 128-byte ones four at a time; wider rows were slower), at most 4
  const uint32_t row = head_dim * uint32_t(dtype_bytes(dtype));
  uint32_t h = 1;
  while (h < 4 && 2 * h * row <= 512 && num_kv_heads % (2 * h) == 0) h *= 2;
  return h;
}

hipError_t launch_decode_partitions(int dtype, uint32_t head_dim, const DecodeKernelArgs& a,
                                    uint64_t num_workgroups, hipStream_t stream) {
  const hipError_t e = launch_order(a, stream);
  if (e != hipSuccess) return e;
  switch (dtype) {
    case kF32: return launch_decode_f32(head_dim, a, num_workgroups, stream);
    case kF16: return launch_decode_f16(head_dim, a, num_workgroups, stream);
    case kBF16: return launch_decode_bf16(head_dim, a, num_workgroups, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_reduce(int dtype, const ReduceKernelArgs& a, hipStream_t stream) {
  const uint64_t waves = uint64_t(a.num_seqs) * a.num_q_heads;
  const uint32_t blocks = uint32_t((waves + kWaves - 1) / kWaves);
  switch (dtype) {
    case kF32:
      hipLaunchKernelGGL(decode_reduce_kernel<kF32>, dim3(blocks), dim3(kThreads), 0, stream, a);
      break;
    case kF16:
      hipLaunchKernelGGL(decode_reduce_kernel<kF16>, dim3(blocks), dim3(kThreads), 0, stream, a);
      break;
    case kBF16:
      hipLaunchKernelGGL(decode_reduce_kernel<kBF16>, dim3(blocks), dim3(kThreads), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#endif  // HPKV_DECODE_HAS(0)

}  // namespace hpkv
