// Shared device helpers for the SPD kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spd.h"

namespace spd {

typedef uint16_t bf16;  // bfloat16 bit pattern
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float((uint32_t)v << 16); }

// float -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return f2bf(v); }

// ---------------------------------------------------------------------------
// MFMA operand traits.  A 16x16 output tile per wave; lane l holds operand rows
// (A) or columns (B) l%16 and the k-group l/16.  The hardware pairs A and B
// elements by the same (lane group, element) slot, so any fixed map from slots
// to k is a valid reduction order as long as A and B use the same map; every
// kernel here loads KPL consecutive k per lane at offset (l/16)*KPL.
// Output: lane l holds D[4*(l/16)+i][l%16], i = 0..3.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 32;  // k per instruction
  static constexpr int KPL = 8;     // k per lane
  typedef uint4 frag;
  static __device__ __forceinline__ frag zero() { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                   __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
  }
  // pack 8 floats (rounded to bf16) into one fragment
  static __device__ __forceinline__ frag pack(const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ frag zero() { return 0.f; }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const float* v) { return v[0]; }
};

// ---------------------------------------------------------------------------
// Wave reductions (xor butterflies; every lane ends with the result)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, WAVE);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, WAVE);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// (value, index) maximum with the lowest index winning ties; NaN never wins.
struct ArgMax {
  float v;
  int i;
};
__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgMax b;
    b.v = __shfl_xor(a.v, o, WAVE);
    b.i = __shfl_xor(a.i, o, WAVE);
    a = argmax_merge(a, b);
  }
  return a;
}
constexpr int ARG_NONE = 0x7fffffff;

// exact integer weight of an fp32 probability: floor(p * 2^52); <= 0 or NaN -> 0
__device__ __forceinline__ uint64_t prob_weight(float p) {
  return (p > 0.f) ? (uint64_t)((double)p * 4503599627370496.0) : 0ull;
}

// floor(u * S / 2^32) for a 32-bit u and 64-bit S
__device__ __forceinline__ uint64_t scale_u32(uint32_t u, uint64_t S) {
  uint64_t lo = (uint64_t)u * (S & 0xffffffffull);
  uint64_t hi = (uint64_t)u * (S >> 32);
  return hi + (lo >> 32);
}

}  // namespace spd
