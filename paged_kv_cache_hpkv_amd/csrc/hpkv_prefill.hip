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
//    tile ahead of use and fetch K and V rows one tile ahead of the product
//    into a double-buffered LDS tile (one barrier per tile): at head_dim 128
//    with direct-to-LDS loads into XOR-swizzled rows, otherwise with 16-byte
//    loads staged through registers into padded rows.
//  * S^T = K Q^T with v_mfma_f32_16x16x32 (A = K rows from LDS, B = q held in
//    registers for the whole loop; lane layout A[l%16][8(l/16)+e],
//    B[8(l/16)+e][l%16], D[4(l/16)+r][l%16]). Lane l ends with keys
//    16u+4(l/16)+r of row l%16 of its column block.
//  * Causal mask (key <= position) and online softmax in base 2 per row (the
//    scale times log2(e) enters in the exponent's FMA), with a lazy rescale:
//    each lane tests the max of its own scores against the row's threshold,
//    and the row max is exchanged among the four lanes holding the row only
//    when a rescale is due.
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
#include <float.h>
#include <math.h>

#include <type_traits>

#include "hpkv_device.h"

namespace hpkv {
namespace {

constexpr int kWave = 64;
constexpr int kKeyTile = 32;  // keys per tile (one 16x16x32 contraction of P.V)
constexpr uint32_t kSegKeys = 4096;  // keys whose pool rows a workgroup resolves at once

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

// Maximum of two scores as IEEE maximum (a NaN operand gives NaN): gfx950's
// v_maximum3_f32, which needs none of the quieting instructions an fmaxf of
// matrix-core results costs. The row max only shifts the exponent; a NaN score
// makes its row NaN under either maximum.
__device__ inline float smax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// Max over the four lanes l, l^16, l^32, l^48 that hold one row of a score tile
// (v_permlane32_swap / v_permlane16_swap exchange whole 32- and 16-lane halves).
__device__ inline float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return smax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two fp32 weights rounded to nearest even in the 16-bit input type, packed low-first.
template <int DT>
__device__ inline uint32_t pack16(float x, float y) {
  uint32_t r;
  if constexpr (DT == kBF16) {
    const bf16x2 v = bf16x2{(__bf16)x, (__bf16)y};
    __builtin_memcpy(&r, &v, 4);
  } else {
    const f16x2 v = f16x2{(_Float16)x, (_Float16)y};
    __builtin_memcpy(&r, &v, 4);
  }
  return r;
}

template <int DT>
__device__ inline uint32_t nan_bits16() {
  return DT == kBF16 ? 0x7fc0u : 0x7e00u;
}

template <int DT, int D, int JT, int NW, int MINB, typename Idx>
__global__ __launch_bounds__(NW * kWave, MINB) void prefill_mfma_kernel(const PrefillKernelArgs a) {
  static_assert(DT != kF32 && D % 32 == 0 && D <= 256, "unsupported shape");
  constexpr int NTH = NW * kWave;
  constexpr int CPR = D * 2 / 16;                       // 16-byte chunks per K/V row
  constexpr int LOADERS = NTH < kKeyTile * CPR ? NTH : kKeyTile * CPR;
  constexpr int RPP = LOADERS / CPR;                    // tile rows per load pass
  constexpr int NP = kKeyTile / RPP;                    // load passes per tile
  static_assert(kKeyTile % RPP == 0 && LOADERS % CPR == 0, "load mapping");
  // head_dim 128: K/V tiles arrive by direct-to-LDS loads into unpadded rows whose 16-byte
  // chunks are XOR-swizzled by row (see dma_kv); other head sizes stage the tiles through
  // registers into padded rows (16-byte K reads and transposed 8-byte V reads on distinct
  // banks either way).
  constexpr bool DL = D == 128;
  constexpr int KROW = DL ? D * 2 : D * 2 + 16;  // LDS bytes per K row
  constexpr int VROW = DL ? D * 2 : D * 2 + 32;  // LDS bytes per V row
  constexpr int KS = D / 32;        // k-steps of the score product
  constexpr int NB = D / 16;        // 16-column blocks of O^T
  constexpr int ROWS = NW * 16 * JT;

  // the two buffers of the double-buffered tile are separate LDS objects, so the compiler
  // can tell a direct-to-LDS load into one from a read of the other and need not wait for
  // the load before the read
  __shared__ __attribute__((aligned(16))) char s_k0[kKeyTile * KROW];
  __shared__ __attribute__((aligned(16))) char s_k1[kKeyTile * KROW];
  __shared__ __attribute__((aligned(16))) char s_v0[kKeyTile * VROW];
  __shared__ __attribute__((aligned(16))) char s_v1[kKeyTile * VROW];
  __shared__ uint32_t s_rows[kSegKeys];  // pool row of each key of the current segment

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid % kWave;
  const uint32_t wave = tid / kWave;
  const uint32_t q4 = lane / 16;   // lane quarter
  const uint32_t col = lane % 16;  // MFMA column: row of the wave's column block

  // XCD-aware work item: the grid is a multiple of 8 and block b runs on XCD b % 8.
  const uint32_t per_xcd = gridDim.x / 8;
  const uint32_t work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= a.num_work) return;
  const uint32_t pb = a.pos_blocks - 1 - work % a.pos_blocks;  // a sequence's longest first
  const uint32_t sg = work / a.pos_blocks;
  const uint32_t s = sg % a.num_seqs;
  const uint32_t g = sg / a.num_seqs;
  const uint32_t G = a.group;
  const uint32_t QP = a.block_positions;

  const int64_t c0 = a.cu_q[s];
  const int64_t c1 = a.cu_q[s + 1];
  const int32_t pstart = a.q_start[s];
  const Idx* seq_ptr = static_cast<const Idx*>(a.seq_ptr);
  const Idx* block_table = static_cast<const Idx*>(a.block_table);
  const uint64_t first = seq_ptr[s];
  const uint64_t last = seq_ptr[s + 1];
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

  // Scores are scaled by c = |scale| * log2(e) >= 0; a negative scale is folded into q
  // as a sign flip (exact), so the row max of the raw products is the max of the scores.
  const float c = fmaxf(fabsf(a.scale_log2), FLT_MIN);  // > 0 (a zero scale acts as FLT_MIN)
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  // lazy rescaling: the subtracted max is only raised when the row max grows by more
  // than 8 (log2 units), so weights stay below 2^8 and most tiles skip the rescale
  const float thr = c > 0.0f ? 8.0f / c : INFINITY;

  // rows of this lane: position (or -1 if inactive) and the query row in q/out
  int32_t pos[JT];
  uint64_t qrow[JT];
  u32x4 qop[JT][KS];
  int32_t min_pos = 0x7fffffff;  // smallest active position of this lane
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const uint32_t r = wave * 16 * JT + jt * 16 + col;
    const uint32_t pl = p_lo + r / G;
    const bool active = r < QP * G && pl < p_hi;
    pos[jt] = active ? int32_t(uint32_t(pstart) + pl) : -1;
    if (active) min_pos = min(min_pos, pos[jt]);
    qrow[jt] = active ? (uint64_t(c0 + pl) * a.num_q_heads + uint64_t(g) * G + r % G) : 0;
    const char* qp = static_cast<const char*>(a.q) + (qrow[jt] * D_ + 8 * q4) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = active ? *reinterpret_cast<const u32x4*>(qp + 64 * ks) : u32x4{0, 0, 0, 0};
      qop[jt][ks] = v ^ qflip;
    }
  }
  // tiles wholly at or below the wave's smallest active position need no causal mask
#pragma unroll
  for (int o = 32; o >= 1; o /= 2) min_pos = min(min_pos, __shfl_xor(min_pos, o));
  const bool wave_active = min_pos != 0x7fffffff;

  f32x4 acc[JT][NB];
  f32x4 accl[JT];         // row sums of the weights (the matrix cores add them up)
  float mthr[JT], mc[JT]; // rescale threshold (raw units) and the subtracted max * c
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    mthr[jt] = -INFINITY;
    mc[jt] = 0.0f;
    accl[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[jt][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const uint32_t one2 = DT == kBF16 ? 0x3f803f80u : 0x3c003c00u;  // two 16-bit 1.0s
  const u32x4 ones = u32x4{one2, one2, one2, one2};

  // loader role: tile row lr (+ RPP per pass), 16-byte chunk lc
  const bool loader = tid < uint32_t(LOADERS);
  const uint32_t lr = tid / CPR, lc = tid % CPR;
  const uint64_t row_stride = uint64_t(a.num_kv_heads) * D_ * 2;
  const uint64_t head_off = uint64_t(g) * D_ * 2 + lc * 16;
  const char* kbase = static_cast<const char*>(a.k_cache) + head_off;
  const char* vbase = static_cast<const char*>(a.v_cache) + head_off;
  bool bad_page = false;
  u32x4 kr[NP], vr[NP];
  auto load_kv = [&](uint32_t tl) {  // tl: first key of the tile, relative to the segment
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint64_t off = uint64_t(s_rows[tl + p * RPP + lr]) * row_stride;
      kr[p] = load16<false>(kbase + off);
      vr[p] = load16<false>(vbase + off);
    }
  };
  auto store_lds = [&](int b) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t r = p * RPP + lr;
      *reinterpret_cast<u32x4*>(&(b ? s_k1 : s_k0)[r * KROW + lc * 16]) = kr[p];
      *reinterpret_cast<u32x4*>(&(b ? s_v1 : s_v0)[r * VROW + lc * 16]) = vr[p];
    }
  };
  // Direct-to-LDS tile load (head_dim 128): 16 lanes per 256-byte row, so one wave's
  // global_load_lds_dwordx4 covers 4 whole rows, and lane i's 16 bytes land at the wave's
  // LDS base + 16 i (the wave's rows are contiguous, unpadded). Lane (lr, lc) fetches the
  // logical chunk that belongs at LDS chunk lc of its row: for K, LDS chunk c of tile row
  // r holds logical chunk c ^ (r & 15), so the 16 rows of a K operand read at one logical
  // chunk sit on distinct banks; for V, c ^ 2 (r & 7), which permutes whole 32-byte pairs,
  // so the four rows of a transposed V read (two 8-byte pieces of one pair each) do.
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint64_t dl_head = uint64_t(g) * D_ * 2;
  const char* kdl = static_cast<const char*>(a.k_cache) + dl_head + (lc ^ (lr & 15u)) * 16u;
  const char* vdl = static_cast<const char*>(a.v_cache) + dl_head + (lc ^ (2u * (lr & 7u))) * 16u;
  auto dma_kv = [&](uint32_t tl, auto buf_tag) {
    constexpr int b = decltype(buf_tag)::value;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint64_t off = uint64_t(s_rows[tl + p * RPP + lr]) * row_stride;
      const uint32_t r0 = p * RPP + 4 * wave_u;  // first of the wave's four rows
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)(kdl + off),
          (__attribute__((address_space(3))) void*)(&(b ? s_k1 : s_k0)[r0 * KROW]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (__attribute__((address_space(1))) void*)(vdl + off),
          (__attribute__((address_space(3))) void*)(&(b ? s_v1 : s_v0)[r0 * VROW]), 16, 0, 0);
    }
  };

  // Direct-to-LDS tiles: this lane's byte offsets within a tile buffer of its K operand
  // read at each k-step (row col of a 16-row block) and of its transposed V read for each
  // 16-column block of O^T (the first of the two 16-row halves). Each is one register
  // held across the loop, so every LDS read below is that register plus a constant (the
  // buffer, the row block) that the read instruction carries as its offset. The empty asm
  // keeps the compiler from splitting them back into a row part and a swizzle part that
  // it would add again in every tile.
  uint32_t koff[KS], voff[NB];
  if constexpr (DL) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      koff[ks] = col * KROW + (((4 * ks + q4) ^ col) * 16);
      asm volatile("" : "+v"(koff[ks]));
    }
    const uint32_t vr = 4 * q4 + col / 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      voff[nb] = vr * VROW + 8 * ((col % 4) & 1) + 16 * ((2 * nb + (col % 4) / 2) ^ (2 * (vr & 7)));
      asm volatile("" : "+v"(voff[nb]));
    }
  }

  // One 32-key tile: scores, online softmax, P.V. MASK: some key of the tile lies past
  // the position of some row of this wave (the diagonal tiles); the others skip the mask.
  // buf: the LDS buffer, a compile-time constant on the direct-to-LDS path (each buffer a
  // distinct object in the code), a runtime index otherwise
  auto tile = [&](auto mask_tag, auto buf, uint32_t tb) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int b = int(buf);
    // scores: keys tb + 16u + 4*q4 + r of row `col` of each column block
    f32x4 sacc[2][JT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) sacc[u][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(
            DL ? &(b ? s_k1 : s_k0)[16 * u * KROW + koff[ks]]
               : &(b ? s_k1 : s_k0)[(16 * u + col) * KROW + (32 * ks + 8 * q4) * 2]);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
          sacc[u][jt] = mfma_16x16x32<DT>(kop, qop[jt][ks], sacc[u][jt]);
      }
    }
    u32x4 pop[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = sacc[e / 4][jt][e % 4];
        if constexpr (MASK) {
          if (int32_t(tb + 16 * (e / 4) + 4 * q4 + (e % 4)) > pos[jt]) sv[e] = -INFINITY;
        }
      }
      // this lane's max of its eight scores (four v_maximum3); a row's max exceeds its
      // threshold exactly when the max of one of its four lanes does, so the exchange
      // between the lanes is only needed on the (rare) rescale branch
      const float la = smax(smax(sv[0], sv[1]), sv[2]);
      const float lb = smax(smax(sv[3], sv[4]), sv[5]);
      const float lmax = smax(lb, smax(smax(sv[6], sv[7]), la));
      if (__any(lmax > mthr[jt])) {
        const float mt = row_max4(lmax);
        const bool need = mt > mthr[jt];
        const float mcn = need ? mt * c : mc[jt];
        // no earlier weights on first use (mthr still -inf): the accumulators are zero
        const float corr = mthr[jt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc[jt] - mcn);
        if (need) mthr[jt] = mt + thr;
        mc[jt] = mcn;
        accl[jt] *= corr;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[jt][nb] *= corr;
      }
      // masked scores are -inf and c > 0, so their weight is exactly 0
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], c, -mc[jt]));
      pop[jt] = u32x4{pack16<DT>(pv[0], pv[1]), pack16<DT>(pv[2], pv[3]),
                      pack16<DT>(pv[4], pv[5]), pack16<DT>(pv[6], pv[7])};
    }
    // O^T += V^T P^T; lane (q4, col) fetches row 4*q4 + col/4 (and 16 + that) of the
    // tile, columns 16*nb + 4*(col%4) .. +3, and receives column 16*nb + col.
    const uint32_t vr_row = 4 * q4 + col / 4;
    const char* vrow0 = &(b ? s_v1 : s_v0)[vr_row * VROW + 8 * (col % 4)];
    const char* vbuf = b ? s_v1 : s_v0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint2 lo = lds_read_tr16(DL ? vbuf + voff[nb] : vrow0 + 32 * nb);
      const uint2 hi = lds_read_tr16(DL ? vbuf + 16 * VROW + voff[nb] : vrow0 + 16 * VROW + 32 * nb);
      const u32x4 vop = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) acc[jt][nb] = mfma_16x16x32<DT>(vop, pop[jt], acc[jt][nb]);
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) accl[jt] = mfma_16x16x32<DT>(ones, pop[jt], accl[jt]);
  };

  // Keys are processed in segments of kSegKeys: the workgroup first resolves every key
  // of the segment to its pool row through the block table (keys past the block's last
  // position reuse the last visible key), then streams the segment's tiles.
  for (uint32_t seg0 = 0; seg0 < kend; seg0 += kSegKeys) {
    const uint32_t seg_len = kend - seg0 < kSegKeys ? kend - seg0 : kSegKeys;
    const uint32_t seg_tiles = (seg_len + kKeyTile - 1) / kKeyTile;
    for (uint32_t k = tid; k < seg_tiles * kKeyTile; k += NTH) {
      const uint32_t key = seg0 + k < kend ? seg0 + k : kend - 1;
      const uint32_t pg = fastdiv(key, a.page_div);
      uint64_t ph = uint64_t(block_table[first + pg]);
      if (ph >= a.num_pages) {
        bad_page = true;
        ph = 0;
      }
      s_rows[k] = uint32_t(ph * a.page_size + (key - pg * a.page_size));
    }
    __syncthreads();
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if constexpr (DL) {
      // tile it + 1 streams into the other buffer while tile it is computed; each thread
      // waits for its own loads before the barrier that hands the buffer over
      dma_kv(0, B0{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      auto step = [&](uint32_t it, auto cur, auto nxt) {
        const uint32_t tb = seg0 + it * kKeyTile;
        if (it + 1 < seg_tiles) dma_kv((it + 1) * kKeyTile, nxt);
        if (wave_active) {
          if (int32_t(tb + kKeyTile - 1) <= min_pos) {
            tile(std::false_type{}, cur, tb);
          } else {
            tile(std::true_type{}, cur, tb);
          }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      };
      for (uint32_t it = 0; it < seg_tiles; it += 2) {
        step(it, B0{}, B1{});
        if (it + 1 < seg_tiles) step(it + 1, B1{}, B0{});
      }
    } else {
      if (loader) {
        load_kv(0);
        store_lds(0);
      }
      __syncthreads();
      for (uint32_t it = 0; it < seg_tiles; ++it) {
        const uint32_t tb = seg0 + it * kKeyTile;
        const int b = it & 1;
        const bool has_next = it + 1 < seg_tiles;
        if (loader && has_next) load_kv((it + 1) * kKeyTile);
        if (wave_active) {
          if (int32_t(tb + kKeyTile - 1) <= min_pos) {
            tile(std::false_type{}, b, tb);
          } else {
            tile(std::true_type{}, b, tb);
          }
        }
        if (loader && has_next) store_lds(b ^ 1);
        __syncthreads();
      }
    }
  }

  const bool any_bad = __syncthreads_or(bad_page);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    if (pos[jt] < 0) continue;
    const float inv = any_bad ? __builtin_nanf("") : 1.0f / accl[jt][0];
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

// Launch shape per head size: 16-row column blocks per wave (JT), waves per
// workgroup (NW) and the launch bound's minimum workgroups per CU (MINB).
// Every operand byte read from LDS feeds JT matrix-core products, and the LDS
// read rate (not the matrix cores) bounds a one-block wave, so two blocks per
// wave is the best balance where the registers allow it; at head_dim 256 the
// accumulators of two blocks do not fit two waves per SIMD, so it keeps one
// block per wave and eight waves per workgroup. Every shape covers 128 rows
// per workgroup. The chain scores ->
// softmax -> P.V of one wave is latency-bound, so more waves per SIMD pay: at
// head_dim 128 three workgroups per CU cap the registers at 168, which costs
// four spilled registers stored before the tile loop and reloaded after it
// (three waves per SIMD; LDS 3 x 49 KB). head_dim 32 and 64 need no tighter
// bound: their registers (at most 128) and LDS (at most 36 KB) already let
// four workgroups share a CU, four waves per SIMD.
template <int DT, int D>
struct PrefillShape {
  static constexpr int JT = D >= 256 ? 1 : 2;
  static constexpr int NW = D >= 256 ? 8 : 4;
  static constexpr int MINB = D >= 256 ? 1 : (D == 128 ? 3 : 2);
  static constexpr int ROWS = NW * 16 * JT;
};

template <int DT, int D>
hipError_t launch_prefill_shape(const PrefillKernelArgs& a, uint32_t nwg, hipStream_t stream) {
  using S = PrefillShape<DT, D>;
  if (a.idx64) {
    hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, S::JT, S::NW, S::MINB, uint64_t>), dim3(nwg),
                       dim3(S::NW * kWave), 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, S::JT, S::NW, S::MINB, uint32_t>), dim3(nwg),
                       dim3(S::NW * kWave), 0, stream, a);
  }
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
  static_assert(PrefillShape<kBF16, 256>::ROWS == PrefillShape<kBF16, 128>::ROWS &&
                PrefillShape<kBF16, 32>::ROWS == PrefillShape<kBF16, 128>::ROWS,
                "one row count for every head size");
  (void)head_dim;
  return PrefillShape<kBF16, 128>::ROWS;
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
