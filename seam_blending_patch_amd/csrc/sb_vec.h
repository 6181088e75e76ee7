// sb_vec.h -- storage vectors and fp32 <-> storage conversions for gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sb {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elem { static constexpr int bytes = DT == DT_F32 ? 4 : 2; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A vector of VB bytes of storage held as 32-bit words (VB = 2 keeps one
// 16-bit element in the low half of w[0]).
template <int VB> struct Vec {
  static constexpr int NW = VB >= 4 ? VB / 4 : 1;
  uint32_t w[NW];
};

template <int VB, bool NT>
__device__ __forceinline__ Vec<VB> vload(const char *p) {
  Vec<VB> v;
  if constexpr (VB == 16) {
    u32x4 q = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p))
                 : *reinterpret_cast<const u32x4 *>(p);
    v.w[0] = q.x; v.w[1] = q.y; v.w[2] = q.z; v.w[3] = q.w;
  } else if constexpr (VB == 4) {
    v.w[0] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p))
                : *reinterpret_cast<const uint32_t *>(p);
  } else {
    static_assert(VB == 2, "vector width");
    v.w[0] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p))
                : *reinterpret_cast<const uint16_t *>(p);
  }
  return v;
}

template <int VB, bool NT>
__device__ __forceinline__ void vstore(char *p, const Vec<VB> &v) {
  if constexpr (VB == 16) {
    u32x4 q = {v.w[0], v.w[1], v.w[2], v.w[3]};
    if (NT) __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(p));
    else *reinterpret_cast<u32x4 *>(p) = q;
  } else if constexpr (VB == 4) {
    if (NT) __builtin_nontemporal_store(v.w[0], reinterpret_cast<uint32_t *>(p));
    else *reinterpret_cast<uint32_t *>(p) = v.w[0];
  } else {
    uint16_t h = (uint16_t)v.w[0];
    if (NT) __builtin_nontemporal_store(h, reinterpret_cast<uint16_t *>(p));
    else *reinterpret_cast<uint16_t *>(p) = h;
  }
}

// elements per vector
template <int DT, int VB> struct VecInfo { static constexpr int V = VB / Elem<DT>::bytes; };

// storage bits -> fp32 (exact)
template <int DT> __device__ __forceinline__ float widen(uint32_t bits) {
  if constexpr (DT == DT_F32) return __uint_as_float(bits);
  else if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  else return __uint_as_float(bits << 16);
}

// fp32 -> storage bits, round to nearest even (hardware conversions: v_cvt_f16_f32,
// v_cvt_pk_bf16_f32; fp32 is the identity)
template <int DT> __device__ __forceinline__ uint32_t narrow(float v) {
  if constexpr (DT == DT_F32) return __float_as_uint(v);
  else if constexpr (DT == DT_F16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
  else return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

// RN_T as an fp32 -> fp32 map
template <int DT> __device__ __forceinline__ float rn(float v) {
  if constexpr (DT == DT_F32) return v;
  else return widen<DT>(narrow<DT>(v));
}

template <int DT, int VB>
__device__ __forceinline__ void unpack(const Vec<VB> &v, float *f) {
  constexpr int V = VecInfo<DT, VB>::V;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = __uint_as_float(v.w[k]);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = widen<DT>((v.w[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu);
  }
}

template <int DT, int VB>
__device__ __forceinline__ Vec<VB> pack(const float *f) {
  constexpr int V = VecInfo<DT, VB>::V;
  Vec<VB> v;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int k = 0; k < V; ++k) v.w[k] = __float_as_uint(f[k]);
  } else if constexpr (V == 1) {
    v.w[0] = narrow<DT>(f[0]);
  } else {
#pragma unroll
    for (int k = 0; k < V; k += 2) v.w[k >> 1] = narrow<DT>(f[k]) | (narrow<DT>(f[k + 1]) << 16);
  }
  return v;
}

} // namespace sb

namespace sb {

// ---------------------------------------------------------------------------
// Packed pairs of 16-bit storage values (two elements per 32-bit word)
// ---------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// exact widening of a packed pair
template <int DT> __device__ __forceinline__ f32x2 widen2(uint32_t w) {
  if constexpr (DT == DT_F16) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  } else {
    f32x2 r;
    r.x = __uint_as_float(w << 16);
    r.y = __uint_as_float(w & 0xFFFF0000u);
    return r;
  }
}

// both lanes rounded to nearest even with one conversion (v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32)
template <int DT> __device__ __forceinline__ uint32_t narrow2(f32x2 v) {
  if constexpr (DT == DT_F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// RN_T(a + b) of two packed pairs.  For binary16 the addition is done in
// binary16 (v_pk_add_f16), which equals rounding the exact sum to fp32 and
// then to binary16 (fp32 has at least 2p + 2 bits, so the double rounding is
// innocuous); for bfloat16 it is an fp32 add and one packed conversion.
template <int DT> __device__ __forceinline__ uint32_t add2(uint32_t a, uint32_t b) {
  if constexpr (DT == DT_F16) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
  } else {
    const f32x2 fa = widen2<DT>(a), fb = widen2<DT>(b);
    f32x2 s;
    s.x = fa.x + fb.x;
    s.y = fa.y + fb.y;
    return narrow2<DT>(s);
  }
}

} // namespace sb
