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
//  * One workgroup (4 waves) per (sequence, KV head, query-head tile,
//    context partition of part_tokens tokens). All query heads of the tile
//    are served from one pass over the partition's K and V, so a GQA group
//    reads its KV once.
//  * The workgroup first resolves every token of its partition to a pool row
//    through the block table and keeps the row offsets in LDS; the token
//    loop then needs no division and no table reads.
//  * A 16-byte vector load per lane; a token row of head_dim elements is
//    covered by LPR = head_dim*bytes/16 adjacent lanes, so one wave load
//    fetches RPL = 64/LPR whole rows (coalesced 2x128 B per 256 B row at
//    d=128 bf16). Each wave keeps 8 K and 8 V loads in flight per tile.
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
#include <math.h>

#include "hpkv_internal.h"

namespace hpkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

template <int DT>
struct Elem {
  static constexpr int bytes = DT == kF32 ? 4 : 2;
};

// Reinterprets a 32-bit word as a pair of 16-bit floats. (Written with memcpy:
// hipcc 7.2 miscompiles __builtin_bit_cast applied to an element of an
// ext_vector_type value, reading element 0 instead.)
template <typename V>
__device__ inline V as_pair(uint32_t w) {
  V r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}

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

// Widens one 16-byte chunk to 16/bytes floats.
template <int DT>
__device__ inline void widen16(const u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = as_pair<f16x2>(w[i]);
      f[2 * i] = float(h.x);
      f[2 * i + 1] = float(h.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
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

// Round-to-nearest-even conversion of fp32 to the storage type.
template <int DT>
__device__ inline void store_out(void* out, uint64_t idx, float x) {
  if constexpr (DT == kBF16) {
    uint32_t u = __float_as_uint(x);
    uint16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      r = 0x7fc0;  // NaN
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
      r = uint16_t(u >> 16);
    }
    static_cast<uint16_t*>(out)[idx] = r;
  } else if constexpr (DT == kF16) {
    static_cast<_Float16*>(out)[idx] = _Float16(x);
  } else {
    static_cast<float*>(out)[idx] = x;
  }
}

// 16-byte global load; non-temporal loads stream K/V past the caches.
template <bool NONTEMPORAL>
__device__ inline u32x4 load16(const char* p) {
  const u32x4* v = reinterpret_cast<const u32x4*>(p);
  if constexpr (NONTEMPORAL) {
    return __builtin_nontemporal_load(v);
  } else {
    return *v;
  }
}

__device__ inline uint32_t fastdiv(uint32_t n, FastDiv d) {
  return uint32_t((uint64_t(n) * d.mul) >> d.shift);
}

__device__ inline uint64_t read_idx(const void* p, uint64_t i, int idx64) {
  return idx64 ? static_cast<const uint64_t*>(p)[i] : static_cast<const uint32_t*>(p)[i];
}

// The sequence-level checks the reduce kernel can also make (it sees only
// context_lens): a negative length or one above max_context_len.
__device__ inline bool length_is_bad(int32_t n, uint32_t max_context_len) {
  return n < 0 || uint32_t(n) > max_context_len;
}

__device__ inline uint32_t num_parts(int32_t n, uint32_t part_tokens) {
  return n <= 0 ? 1u : (uint32_t(n) + part_tokens - 1) / part_tokens;
}

template <int DT, int D, int GT, class TU>
__global__ __launch_bounds__(TU::NW * 64, TU::MINW) void decode_partition_kernel(
    const DecodeKernelArgs a) {
  constexpr int NW = TU::NW;
  constexpr int NTH = NW * kWave;    // threads per workgroup
  constexpr int NLOAD = TU::NLOAD;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int EPL = 16 / EB;       // elements per 16-byte chunk
  constexpr int CPR = D / EPL;       // chunks per token row
  constexpr int CPL = TU::CPL < CPR ? TU::CPL : CPR;  // chunks per lane
  constexpr int LPR = CPR / CPL;     // lanes per token row
  constexpr int RPL = kWave / LPR;   // token rows per wave load
  constexpr int TT = RPL * NLOAD;    // tokens per wave tile
  constexpr int VPL = CPL * EPL;     // elements of a row per lane
  static_assert(CPR % CPL == 0 && LPR <= kWave && (LPR & (LPR - 1)) == 0,
                "unsupported head_dim");

  __shared__ uint64_t s_row[kMaxPartTokens];
  __shared__ float s_m[NW][GT];
  __shared__ float s_l[NW][GT];
  __shared__ float s_acc[NW][GT][D];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid % kWave;
  const uint32_t wave = tid / kWave;

  uint32_t bid = blockIdx.x;
  const uint32_t ht = bid % a.head_tiles;
  bid /= a.head_tiles;
  const uint32_t part = bid % a.max_parts;
  const uint32_t s = bid / a.max_parts;
  const uint32_t tiles_per_group = a.group / GT;
  const uint32_t g = ht / tiles_per_group;
  const uint32_t h0 = g * a.group + (ht % tiles_per_group) * GT;

  const int32_t n = a.context_lens[s];
  const uint32_t nparts = num_parts(n, a.part_tokens);
  if (part >= nparts) return;

  const uint64_t out_row0 = uint64_t(s) * a.num_q_heads + h0;  // first (s, h) row of the tile
  if (length_is_bad(n, a.max_context_len)) {
    if (part == 0)
      for (uint32_t i = tid; i < GT * D; i += NTH) store_out<DT>(a.out, out_row0 * D + i, NAN);
    return;
  }

  const uint64_t first = read_idx(a.seq_ptr, s, a.idx64);
  const uint64_t last = read_idx(a.seq_ptr, uint64_t(s) + 1, a.idx64);
  bool bad = first > last || last > a.block_table_len ||
             uint64_t(n) > (last - first) * uint64_t(a.page_size);

  const uint32_t p0 = part * a.part_tokens;
  const uint32_t cnt = bad || n == 0 ? 0u : min(uint32_t(n) - p0, a.part_tokens);

  // Resolve each token of the partition to its pool row (element offset of
  // head g's row), once per workgroup.
  int bad_page = 0;
  for (uint32_t i = tid; i < cnt; i += NTH) {
    const uint32_t t = p0 + i;
    const uint32_t lp = fastdiv(t, a.page_div);
    const uint32_t off = t - lp * a.page_size;
    uint64_t phys = read_idx(a.block_table, first + lp, a.idx64);
    if (phys >= a.num_pages) {
      bad_page = 1;
      phys = 0;
    }
    s_row[i] = ((phys * a.page_size + off) * a.num_kv_heads + g) * uint64_t(D);
  }
  bad = __syncthreads_or(bad_page) != 0 || bad;

  if (bad) {  // malformed index buffers: NaN result for this partition
    if (nparts == 1) {
      for (uint32_t i = tid; i < GT * D; i += NTH)
        store_out<DT>(a.out, out_row0 * D + i, NAN);
    } else {
      for (uint32_t i = tid; i < GT * D; i += NTH) {
        const uint64_t r = (out_row0 + i / D) * a.max_parts + part;
        a.ws_o[r * D + i % D] = NAN;
        if (i % D == 0) a.ws_ml[r] = make_float2(NAN, NAN);
      }
    }
    return;
  }

  const uint32_t row = lane / LPR;  // which row of a wave load this lane reads
  const uint32_t c = lane % LPR;    // lane's chunks of that row: j*LPR + c, j < CPL

  u32x4 qv[GT][CPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const char* qp = static_cast<const char*>(a.q) +
                       ((out_row0 + hh) * D + (j * LPR + c) * EPL) * EB;
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

  const char* kbase = static_cast<const char*>(a.k_cache) + c * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + c * 16;

  for (uint32_t tb = wave * TT; tb < cnt; tb += NW * TT) {
    u32x4 kr[NLOAD][CPL], vr[NLOAD][CPL];
#pragma unroll
    for (int k = 0; k < NLOAD; ++k) {
      const uint32_t li = tb + k * RPL + row;
      const uint64_t off = s_row[li < cnt ? li : cnt - 1] * EB;
#pragma unroll
      for (int j = 0; j < CPL; ++j) kr[k][j] = load16<TU::NT>(kbase + off + j * LPR * 16);
#pragma unroll
      for (int j = 0; j < CPL; ++j) vr[k][j] = load16<TU::NT>(vbase + off + j * LPR * 16);
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
        const float z = row_sum<LPR>(part_dot) * a.scale_log2;
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
          s_acc[wave][hh][(j * LPR + c) * EPL + e] = acc[hh][j * EPL + e];
      }
      if (c == 0) {
        s_m[wave][hh] = m[hh];
        s_l[wave][hh] = l[hh];
      }
    }
  }
  __syncthreads();

  // Merge the waves and write the result or the partial.
  for (uint32_t i = tid; i < GT * D; i += NTH) {
    const uint32_t hh = i / D, e = i % D;
    float mx = s_m[0][hh];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_m[w][hh]);
    const float mref = mx == -INFINITY ? 0.0f : mx;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][hh] - mref);
      L = fmaf(s_l[w][hh], f, L);
      O = fmaf(s_acc[w][hh][e], f, O);
    }
    if (nparts == 1) {
      store_out<DT>(a.out, (out_row0 + hh) * D + e, L > 0.0f ? O / L : 0.0f);
    } else {
      const uint64_t r = (out_row0 + hh) * a.max_parts + part;
      a.ws_o[r * D + e] = O;
      if (e == 0) a.ws_ml[r] = make_float2(mx, L);
    }
  }
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
  // global max over partitions
  float mx = -INFINITY;
  for (uint32_t j = lane; j < nparts; j += kWave) mx = fmaxf(mx, ml[j].x);
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sft));
  // total weight
  float L = 0.0f;
  for (uint32_t j = lane; j < nparts; j += kWave) {
    const float2 v = ml[j];
    L = fmaf(v.y, __builtin_amdgcn_exp2f(v.x - mx), L);
  }
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) L += __shfl_xor(L, sft);
  // weighted sum of the partial vectors, partitions in order
  for (uint32_t e = lane; e < a.head_dim; e += kWave) {
    float O = 0.0f;
    for (uint32_t j = 0; j < nparts; ++j)
      O = fmaf(o[uint64_t(j) * a.head_dim + e], __builtin_amdgcn_exp2f(ml[j].x - mx), O);
    store_out<DT>(a.out, sh * a.head_dim + e, O / L);
  }
}

// Launch shapes measured on MI355X (bf16, d=128): for one query head per KV
// head the kernel streams at the HBM ceiling with 8 row loads per lane in
// flight; wider GQA tiles are VALU-heavy and run best with fewer loads per
// tile and the register budget capped for 4 waves per SIMD.
template <int DT, int D, int GT>
struct DefaultTune {
  using type = Tune<4, GT == 1 ? 8 : 4, true, GT >= 8 ? 2 : 4>;
};

template <int DT, int D, int GT>
hipError_t launch_pd(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  using TU = typename DefaultTune<DT, D, GT>::type;
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, GT, TU>), dim3(uint32_t(nwg)),
                     dim3(TU::NW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_d(const DecodeKernelArgs& a, uint64_t nwg, hipStream_t stream) {
  switch (heads_per_workgroup(a.group)) {
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

}  // namespace

uint32_t heads_per_workgroup(uint32_t group) {
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

hipError_t launch_decode_partitions(int dtype, uint32_t head_dim, const DecodeKernelArgs& a,
                                    uint64_t num_workgroups, hipStream_t stream) {
  switch (dtype) {
    case kF32: return launch_dt<kF32>(head_dim, a, num_workgroups, stream);
    case kF16: return launch_dt<kF16>(head_dim, a, num_workgroups, stream);
    case kBF16: return launch_dt<kBF16>(head_dim, a, num_workgroups, stream);
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

}  // namespace hpkv
