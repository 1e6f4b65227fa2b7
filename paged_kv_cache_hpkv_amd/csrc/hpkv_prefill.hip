// Causal chunked-prefill attention over the paged cache for gfx950 (CDNA4).
//
// What is computed ("Paged KV Cache · AI infra interview lesson": section
// "Step 1: slot_mapping and store_kvcache" for chunks that start part-way
// into a page after a prefix hit or an earlier chunk, section "Step 2:
// paged_attention_decode" for the gather through the block table): the
// chunk of sequence s holds query rows i = cu_q[s] .. cu_q[s+1]-1 at
// positions p = q_start[s] + (i - cu_q[s]); for query head h with KV head
// g = h / (Hq / Hkv)
//   out[i,h,:] = sum_{t <= p} softmax_t(scale * q[i,h,:] . K[t,g,:]) * V[t,g,:]
// with K and V rows of token t read from pool row
// block_table[seq_ptr[s] + t / page_size] * page_size + t % page_size
// ("Block-Paged KV Cache", section "Element lookup through the block
// table"). The chunk's own rows are stored in the pool before this runs.
//
// Design (a dense contraction, 4*d flops per (row, key) pair: matrix cores):
//  * One workgroup of NW waves per (sequence, KV head, block of chunk
//    positions). Its rows are the block's (position, query head) pairs,
//    position-major, with every query head of the GQA group, so each K/V
//    tile staged in LDS feeds all of them. Wave w owns 16*JT consecutive
//    rows as JT column blocks of the transposed score tile.
//  * Key loop over 32-key tiles from token 0 to the block's last position.
//    Loading lanes resolve their key's pool row through the block table one
//    tile ahead of use, fetch K and V rows with 16-byte loads one tile ahead
//    of the product, and write them into a double-buffered LDS tile (one
//    barrier per tile).
//  * S^T = K Q^T with v_mfma_f32_16x16x32 (A = K rows from LDS, B = q held in
//    registers for the whole loop; lane layout A[l%16][8(l/16)+e],
//    B[8(l/16)+e][l%16], D[4(l/16)+r][l%16]). Lane l ends with keys
//    16u+4(l/16)+r of row l%16 of its column block.
//  * Causal mask (key <= position) and online softmax in base 2 per row
//    (scores pre-multiplied by scale*log2(e)); the row max is shared by the
//    four lanes holding the row.
//  * O^T = V^T P^T. The contraction index k = 8(l/16)+e is mapped to key
//    16(e/4)+4(l/16)+(e%4), where the scores already sit, so P needs no data
//    movement. V^T comes straight from the row-major LDS tile through the
//    transposing LDS read ds_read_b64_tr_b16: within each group of 16 lanes,
//    lanes 4r..4r+3 fetch the 16 elements of row r of a 4x16 block and lane i
//    receives column i of the four rows. P is rounded to the input type for
//    the matrix cores and the softmax denominator sums the rounded weights.
//  * Workgroup ids are spread over the 8 XCDs round-robin by the hardware;
//    each XCD is given a contiguous range of work items (position block
//    fastest, then sequence, then KV head), so the blocks of one sequence and
//    neighbouring sequences (which may alias prefix pages) share that XCD's L2.
//  * Keys past the block's last position are never loaded (lanes reuse the
//    last valid key) and masked keys have weight exactly 0, so garbage in
//    unused pool rows cannot reach the accumulators. A malformed sequence
//    (bad cu_q / q_start / seq_ptr entries, a chunk longer than max_q_len or
//    past its slice) gets NaN rows; a block that meets a page id >= num_pages
//    writes NaN rows. Nothing is read or written out of bounds.
#include <math.h>

#include "hpkv_device.h"

namespace hpkv {
namespace {

constexpr int kWave = 64;
constexpr int kKeyTile = 32;  // keys per tile (one 16x16x32 contraction of P.V)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16 at LDS address p (8-byte aligned); returns the four
// 16-bit results of this lane packed in two words.
__device__ inline uint2 lds_read_tr16(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((lds_char*)(const_cast<char*>(p))));
  uint2 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

template <int DT>
__device__ inline uint32_t nan_bits16() {
  return DT == kBF16 ? 0x7fc0u : 0x7e00u;
}

template <int DT, int D, int JT, int NW>
__global__ __launch_bounds__(NW * kWave, 1) void prefill_mfma_kernel(const PrefillKernelArgs a) {
  static_assert(DT != kF32 && D % 32 == 0 && D <= 256, "unsupported shape");
  constexpr int NTH = NW * kWave;
  constexpr int CPR = D * 2 / 16;                       // 16-byte chunks per K/V row
  constexpr int LOADERS = NTH < kKeyTile * CPR ? NTH : kKeyTile * CPR;
  constexpr int RPP = LOADERS / CPR;                    // tile rows per load pass
  constexpr int NP = kKeyTile / RPP;                    // load passes per tile
  static_assert(kKeyTile % RPP == 0 && LOADERS % CPR == 0, "load mapping");
  constexpr int KROW = D * 2 + 16;  // LDS bytes per K row: 16-byte lane reads hit distinct banks
  constexpr int VROW = D * 2 + 32;  // LDS bytes per V row: transposed 8-byte reads likewise
  constexpr int KS = D / 32;        // k-steps of the score product
  constexpr int NB = D / 16;        // 16-column blocks of O^T
  constexpr int ROWS = NW * 16 * JT;

  __shared__ __attribute__((aligned(16))) char s_k[2][kKeyTile * KROW];
  __shared__ __attribute__((aligned(16))) char s_v[2][kKeyTile * VROW];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid % kWave;
  const uint32_t wave = tid / kWave;
  const uint32_t q4 = lane / 16;   // lane quarter
  const uint32_t col = lane % 16;  // MFMA column: row of the wave's column block

  // XCD-aware work item: the grid is a multiple of 8 and block b runs on XCD b % 8.
  const uint32_t per_xcd = gridDim.x / 8;
  const uint32_t work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= a.num_work) return;
  const uint32_t pb = work % a.pos_blocks;
  const uint32_t sg = work / a.pos_blocks;
  const uint32_t s = sg % a.num_seqs;
  const uint32_t g = sg / a.num_seqs;
  const uint32_t G = a.group;
  const uint32_t QP = a.block_positions;

  const int64_t c0 = a.cu_q[s];
  const int64_t c1 = a.cu_q[s + 1];
  const int32_t pstart = a.q_start[s];
  const uint64_t first = read_idx(a.seq_ptr, s, a.idx64);
  const uint64_t last = read_idx(a.seq_ptr, s + 1, a.idx64);
  const int64_t n = c1 - c0;
  bool bad = c0 < 0 || n < 0 || uint64_t(c1) > a.num_q_tokens || n > int64_t(a.max_q_len) ||
             pstart < 0 || last < first || last > a.block_table_len;
  if (!bad) {
    const uint64_t end = uint64_t(pstart) + uint64_t(n);
    bad = end > 0x7fffffffull || end > (last - first) * a.page_size;
  }
  const uint64_t D_ = D;
  if (bad) {
    // every row of the sequence (for this KV head's query heads) becomes NaN
    if (pb != 0) return;
    const int64_t i0 = c0 < 0 ? 0 : c0;
    const int64_t i1 = c1 > int64_t(a.num_q_tokens) ? int64_t(a.num_q_tokens) : c1;
    if (i1 <= i0) return;
    const uint64_t per_row = uint64_t(G) * D_;
    const uint64_t total = uint64_t(i1 - i0) * per_row;
    uint16_t* out = static_cast<uint16_t*>(a.out);
    for (uint64_t e = tid; e < total; e += NTH) {
      const uint64_t i = uint64_t(i0) + e / per_row;
      out[(i * a.num_q_heads + uint64_t(g) * G) * D_ + e % per_row] = uint16_t(nan_bits16<DT>());
    }
    return;
  }
  const uint32_t p_lo = pb * QP;  // first chunk offset of the block
  if (int64_t(p_lo) >= n) return;
  const uint32_t p_hi = int64_t(p_lo + QP) < n ? p_lo + QP : uint32_t(n);
  const uint32_t kend = uint32_t(pstart) + p_hi;  // keys 0 .. kend-1 are visible to the block
  const uint32_t ntiles = (kend + kKeyTile - 1) / kKeyTile;

  // rows of this lane: position (or -1 if inactive) and the query row in q/out
  int32_t pos[JT];
  uint64_t qrow[JT];
  u32x4 qop[JT][KS];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const uint32_t r = wave * 16 * JT + jt * 16 + col;
    const uint32_t pl = p_lo + r / G;
    const bool active = r < QP * G && pl < p_hi;
    pos[jt] = active ? int32_t(uint32_t(pstart) + pl) : -1;
    qrow[jt] = active ? (uint64_t(c0 + pl) * a.num_q_heads + uint64_t(g) * G + r % G) : 0;
    const char* qp = static_cast<const char*>(a.q) + (qrow[jt] * D_ + 8 * q4) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[jt][ks] = active ? *reinterpret_cast<const u32x4*>(qp + 64 * ks) : u32x4{0, 0, 0, 0};
  }

  f32x4 acc[JT][NB];
  float m[JT], l[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    m[jt] = -INFINITY;
    l[jt] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[jt][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // loader role: tile row lr (+ RPP per pass), 16-byte chunk lc
  const bool loader = tid < uint32_t(LOADERS);
  const uint32_t lr = tid / CPR, lc = tid % CPR;
  const char* kbase = static_cast<const char*>(a.k_cache) + lc * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + lc * 16;
  const uint64_t row_stride = uint64_t(a.num_kv_heads) * D_ * 2;
  const uint64_t head_off = uint64_t(g) * D_ * 2;
  uint64_t phys[NP];
  uint32_t poff[NP];
  bool bad_page = false;
  auto fetch_pages = [&](uint32_t tb) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t key = tb + p * RPP + lr;
      key = key < kend ? key : kend - 1;
      const uint32_t pg = fastdiv(key, a.page_div);
      poff[p] = key - pg * a.page_size;
      phys[p] = read_idx(a.block_table, first + pg, a.idx64);
    }
  };
  u32x4 kr[NP], vr[NP];
  auto load_kv = [&]() {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint64_t ph = phys[p];
      if (ph >= a.num_pages) {
        bad_page = true;
        ph = 0;
      }
      const uint64_t off = (ph * a.page_size + poff[p]) * row_stride + head_off;
      kr[p] = load16<false>(kbase + off);
      vr[p] = load16<false>(vbase + off);
    }
  };
  auto store_lds = [&](int b) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t r = p * RPP + lr;
      *reinterpret_cast<u32x4*>(&s_k[b][r * KROW + lc * 16]) = kr[p];
      *reinterpret_cast<u32x4*>(&s_v[b][r * VROW + lc * 16]) = vr[p];
    }
  };

  if (loader) {
    fetch_pages(0);
    load_kv();
    if (ntiles > 1) fetch_pages(kKeyTile);
    store_lds(0);
  }
  __syncthreads();

  for (uint32_t it = 0; it < ntiles; ++it) {
    const uint32_t tb = it * kKeyTile;
    const int b = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (loader && has_next) {
      load_kv();
      if (it + 2 < ntiles) fetch_pages(tb + 2 * kKeyTile);
    }

    // scores: keys tb + 16u + 4*q4 + r of row `col` of each column block
    f32x4 sacc[2][JT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) sacc[u][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kop =
            *reinterpret_cast<const u32x4*>(&s_k[b][(16 * u + col) * KROW + (32 * ks + 8 * q4) * 2]);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) sacc[u][jt] = mfma_16x16x32<DT>(kop, qop[jt][ks], sacc[u][jt]);
      }
    }

    u32x4 pop[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      float z[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int32_t t = int32_t(tb + 16 * (e / 4) + 4 * q4 + (e % 4));
        z[e] = t <= pos[jt] ? sacc[e / 4][jt][e % 4] * a.scale_log2 : -INFINITY;
      }
      float mt = z[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, z[e]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[jt], mt);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float corr = __builtin_amdgcn_exp2f(m[jt] - mu);
      m[jt] = mn;
      l[jt] *= corr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[jt][nb] *= corr;
      uint32_t pw[4];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t b0 = round16<DT>(__builtin_amdgcn_exp2f(z[e] - mu));
        const uint32_t b1 = round16<DT>(__builtin_amdgcn_exp2f(z[e + 1] - mu));
        psum += widen_bits16<DT>(b0) + widen_bits16<DT>(b1);
        pw[e / 2] = b0 | (b1 << 16);
      }
      l[jt] += psum;
      pop[jt] = u32x4{pw[0], pw[1], pw[2], pw[3]};
    }

    // O^T += V^T P^T; lane (q4, col) fetches row 4*q4 + col/4 (and 16 + that) of the
    // tile, columns 16*nb + 4*(col%4) .. +3, and receives column 16*nb + col.
    const char* vrow0 = &s_v[b][(4 * q4 + col / 4) * VROW + 8 * (col % 4)];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint2 lo = lds_read_tr16(vrow0 + 32 * nb);
      const uint2 hi = lds_read_tr16(vrow0 + 16 * VROW + 32 * nb);
      const u32x4 vop = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) acc[jt][nb] = mfma_16x16x32<DT>(vop, pop[jt], acc[jt][nb]);
    }

    if (loader && has_next) store_lds(b ^ 1);
    __syncthreads();
  }

  const bool any_bad = __syncthreads_or(bad_page);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    // the four lane quarters hold disjoint keys of each row: add their sums
    float lt = l[jt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (pos[jt] < 0) continue;
    const float inv = any_bad ? __builtin_nanf("") : 1.0f / lt;
    char* orow = static_cast<char*>(a.out) + (qrow[jt] * D_ + 4 * q4) * 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 v = acc[jt][nb];
      const uint32_t w0 = bits16<DT>(v[0] * inv) | (bits16<DT>(v[1] * inv) << 16);
      const uint32_t w1 = bits16<DT>(v[2] * inv) | (bits16<DT>(v[3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * nb) = uint2{w0, w1};
    }
  }
}

template <int DT, int D>
struct PrefillShape {
  static constexpr int JT = D >= 256 ? 2 : 4;  // 16-row column blocks per wave
  static constexpr int NW = 4;
  static constexpr int ROWS = NW * 16 * JT;
};

template <int DT, int D>
hipError_t launch_prefill_shape(const PrefillKernelArgs& a, uint32_t nwg, hipStream_t stream) {
  using S = PrefillShape<DT, D>;
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, S::JT, S::NW>), dim3(nwg), dim3(S::NW * kWave),
                     0, stream, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_prefill_dtype(uint32_t head_dim, const PrefillKernelArgs& a, uint32_t nwg,
                                hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_prefill_shape<DT, 32>(a, nwg, stream);
    case 64: return launch_prefill_shape<DT, 64>(a, nwg, stream);
    case 128: return launch_prefill_shape<DT, 128>(a, nwg, stream);
    case 256: return launch_prefill_shape<DT, 256>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool prefill_head_dim_supported(int dtype, uint32_t head_dim) {
  if (dtype != kBF16 && dtype != kF16) return false;
  return head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256;
}

uint32_t prefill_rows_per_workgroup(int dtype, uint32_t head_dim) {
  (void)dtype;
  return head_dim >= 256 ? PrefillShape<kBF16, 256>::ROWS : PrefillShape<kBF16, 128>::ROWS;
}

hipError_t launch_prefill(int dtype, uint32_t head_dim, const PrefillKernelArgs& a,
                          uint32_t num_workgroups, hipStream_t stream) {
  switch (dtype) {
    case kBF16: return launch_prefill_dtype<kBF16>(head_dim, a, num_workgroups, stream);
    case kF16: return launch_prefill_dtype<kF16>(head_dim, a, num_workgroups, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hpkv
