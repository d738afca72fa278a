// MFMA fragment helpers for gfx950 (wave64).
//
// One "k-step" contracts 32 values of k. For a 16x16 output tile, lane l of
// the wave supplies operand row (l % 16) and the 8 consecutive k values
// 8*(l/16) .. 8*(l/16)+7 of the step, for both the A and the B operand.
// Accumulator layout: lane l holds C[4*(l/16) + i][l % 16], i = 0..3.
//   bf16: one v_mfma_f32_16x16x32_bf16 per k-step.
//   fp32: eight v_mfma_f32_16x16x4_f32; instruction j contracts element j of
//         every lane's 8 values, i.e. k in {8g + j : g = 0..3}; over j = 0..7
//         that is the same 32 values.
#pragma once

#include <hip/hip_runtime.h>

#include "dg_common.h"

namespace dg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

template <typename T> struct Frag;

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

template <> struct Frag<bf16_t> {
  using type = bf16x8_t;
  __device__ static inline type load(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
  // streamed-once operands (weights): a nontemporal load
  __device__ static inline type load_nt(const bf16_t* p) {
    const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t*>(p));
    return __builtin_bit_cast(bf16x8_t, v);
  }
  __device__ static inline type zero() {
    type z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = static_cast<__bf16>(0.0f);
    return z;
  }
  __device__ static inline f32x4_t mma(const type& a, const type& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Frag<float> {
  using type = f32x8_t;
  __device__ static inline type load(const float* p) { return *reinterpret_cast<const f32x8_t*>(p); }
  __device__ static inline type load_nt(const float* p) { return load(p); }
  __device__ static inline type zero() {
    type z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = 0.f;
    return z;
  }
  __device__ static inline f32x4_t mma(const type& a, const type& b, f32x4_t c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
};

// store/convert helpers
template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ inline float from_f32<float>(float v) { return v; }

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ inline float to_f32<float>(float v) { return v; }

__device__ inline float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

}  // namespace dg
