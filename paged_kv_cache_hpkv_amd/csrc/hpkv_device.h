// Device helpers shared by the gfx950 kernels: vector types, 16-bit float
// conversions, the 16x16x32 matrix-core product and index reads.
#pragma once

#include "hpkv_internal.h"

namespace hpkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

template <typename V>
__device__ inline V as_vec(const u32x4 w) {
  V r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}

template <int DT>
__device__ inline f32x4 mfma_16x16x32(const u32x4 a, const u32x4 b, const f32x4 c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_vec<bf16x8>(a), as_vec<bf16x8>(b), c, 0, 0,
                                                   0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_vec<f16x8>(a), as_vec<f16x8>(b), c, 0, 0, 0);
  }
}

// Two fp32 values rounded to nearest even in the 16-bit input type and packed, lo in
// the low half: one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950.
template <int DT>
__device__ inline uint32_t pack16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint32_t r;
  if constexpr (DT == kBF16) {
    const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    __builtin_memcpy(&r, &b, 4);
  } else {
    const f16x2 h = __builtin_convertvector(f32x2{lo, hi}, f16x2);
    __builtin_memcpy(&r, &h, 4);
  }
  return r;
}

template <int DT>
__device__ inline float widen_bits16(uint32_t b) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(b << 16);
  } else {
    const uint16_t h16 = uint16_t(b);
    _Float16 h;
    __builtin_memcpy(&h, &h16, 2);
    return float(h);
  }
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

// Bits of fp32 x rounded to nearest even in the 16-bit storage type DT
// (NaN stays NaN).
template <int DT>
__device__ inline uint32_t bits16(float x) {
  if constexpr (DT == kBF16) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  } else {
    const _Float16 h = _Float16(x);
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
  }
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

}  // namespace hpkv
