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
// fp32 -> bf16, round to nearest even (the hardware v_cvt_pk_bf16_f32)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float spd_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 spd_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const spd_f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, spd_bf16x2));
}
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)(pack2_bf16(f, 0.f) & 0xffffu); }

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
  // keep the first `n` of the 8 elements (n <= 0: none), zero the rest
  static __device__ __forceinline__ frag mask_from(frag f, int n) {
    const uint32_t m0 = n >= 2 ? 0xffffffffu : (n == 1 ? 0xffffu : 0u);
    const uint32_t m1 = n >= 4 ? 0xffffffffu : (n == 3 ? 0xffffu : 0u);
    const uint32_t m2 = n >= 6 ? 0xffffffffu : (n == 5 ? 0xffffu : 0u);
    const uint32_t m3 = n >= 8 ? 0xffffffffu : (n == 7 ? 0xffffu : 0u);
    return make_uint4(f.x & m0, f.y & m1, f.z & m2, f.w & m3);
  }
  // pack 8 floats (rounded to bf16) into one fragment
  static __device__ __forceinline__ frag pack(const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(v[2 * i], v[2 * i + 1]);
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
  static __device__ __forceinline__ frag mask_from(frag f, int n) { return n >= 1 ? f : 0.f; }
};

// ---------------------------------------------------------------------------
// Wave reductions.  Within each row of 16 lanes: DPP butterflies (quad_perm,
// half-mirror, mirror), which stay in the VALU; the four row results are then
// combined from readlane values.  Every lane ends with the same result, and the
// summation order is fixed.  Callers run them with the whole wave active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
constexpr int DPP_QUAD_1032 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// sum / max over each row of 16 lanes, result in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<DPP_QUAD_1032>(v);
  v += dpp_f32<DPP_QUAD_2301>(v);
  v += dpp_f32<DPP_HALF_MIRROR>(v);
  v += dpp_f32<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f32<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f32<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v += dpp_u64<DPP_QUAD_1032>(v);
  v += dpp_u64<DPP_QUAD_2301>(v);
  v += dpp_u64<DPP_HALF_MIRROR>(v);
  v += dpp_u64<DPP_MIRROR>(v);
  return lane_u64(v, 0) + lane_u64(v, 16) + lane_u64(v, 32) + lane_u64(v, 48);
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

// ---------------------------------------------------------------------------
// Cross-block hand-off without fences.  On this part an agent-scope fence is a
// whole-L2 writeback + invalidate, which stalls every streaming wave on the
// die.  Data that another block of the same launch will read is therefore
// written and read with agent-scope relaxed atomics, which compile to plain
// vector loads/stores carrying the device-coherence bit (sc1): they bypass the
// die-local caches without flushing them.  A block that wrote such data waits
// for its stores to complete (s_waitcnt) before bumping an arrival counter; the
// block that sees the final count reads everyone's data with sc1 loads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i32(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh_i32(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte coherent load of base + byte offset `off` (base must be the same for the
// whole wave: it becomes a buffer descriptor; `off` < 2^31).  buffer_load_dwordx4
// with the device-coherence bit.
__device__ __forceinline__ float4 ld_coh4(const void* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
__device__ __forceinline__ void st_coh4(float* p, float4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  st_coh_u64(q, __builtin_bit_cast(uint64_t, make_float2(v.x, v.y)));
  st_coh_u64(q + 1, __builtin_bit_cast(uint64_t, make_float2(v.z, v.w)));
}

// 16-byte coherent store at byte offset `off` from a wave-uniform base (one
// buffer_store_dwordx4 with the same cache policy as the st_coh stores)
__device__ __forceinline__ void st_coh4b(void* base, uint32_t off, float4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 16);
}

// Every thread of the block calls this after its st_coh stores.  Returns true in
// exactly one of the `expected` blocks sharing `counter`, after all of them have
// arrived; that block resets the counter to zero for the next use.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == expected - 1;
    if (s_last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return s_last != 0;
}

// Two-level form for thousands of arrivals: blocks of group g = id % ngroups
// count on their own counter (counters 64 bytes apart); the last of each group
// counts on the top counter.  counters: [ngroups + 1] x 16 words.
__device__ __forceinline__ bool arrive_last2(unsigned* counters, unsigned id, unsigned total,
                                             unsigned ngroups) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (ngroups > total) ngroups = total;
    const unsigned g = id % ngroups;
    const unsigned gsize = total / ngroups + (g < total % ngroups ? 1u : 0u);
    unsigned* gc = counters + 16 * g;
    unsigned* top = counters + 16 * ngroups;
    int last = 0;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = 1;
      }
    }
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

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
