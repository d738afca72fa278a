// Shared host/device helpers of libdg (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "dg.h"

namespace dg {

// ------------------------------------------------------------------ errors
// Thread-local message of the last failing call (see dg_last_error).
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int hip_check(hipError_t e, const char* what);

#define DG_HIP(call)                                   \
  do {                                                 \
    hipError_t e__ = (call);                           \
    if (e__ != hipSuccess) return ::dg::hip_check(e__, #call); \
  } while (0)

#define DG_LAUNCH_CHECK(what) \
  do { hipError_t e__ = hipGetLastError(); if (e__ != hipSuccess) return ::dg::hip_check(e__, what); } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// FP8 (E4M3) codes and float32 per-row scales of one layer's routed experts: gate/up codes in the
// paired-tile order of tiles.h (per expert gw * F * D bytes), down codes (per expert D * F bytes),
// scales [E][gw][F] and [E][D].
struct ExpertsFp8 {
  const uint8_t* gu;
  const uint8_t* dn;
  const float* s_gu;
  const float* s_dn;
};

// -------------------------------------------------------------- bf16 bits
// bf16 is handled as raw 16-bit patterns (upper half of an fp32).
typedef uint16_t bf16_t;

__host__ __device__ inline float bf16_to_f32(bf16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

// round to nearest even (inputs are finite in this library)
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ inline float bf16lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ inline float bf16hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; same bits as f32_to_bf16
// for finite values
typedef __bf16 bf16x2_native_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_native_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------ wave64 reductions
template <typename T>
__device__ inline T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, 64); }

// Partner exchanges without the LDS permute network. Inside a 16-lane row, DPP moves: quad_perm
// [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (lane i <-> 7 - i within
// 8: pairs the two quads of a half-row) and row_mirror (i <-> 15 - i: pairs the two halves). Across
// rows, the gfx950 row swaps: v_permlane16_swap / v_permlane32_swap given the same register twice
// return, in one of their two results, the value of the partner row (l ^ 16, l ^ 32). A symmetric
// combine op(x, partner) at each of the six levels reduces the whole wave, and since op is
// commutative every lane ends with the same bits.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }

// partner value in the other 16-lane row of the 32-lane half (lane ^ 16) / other half (lane ^ 32)
__device__ inline uint32_t xrow16_u32(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? a[0] : a[1];
}
__device__ inline uint32_t xrow32_u32(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? a[0] : a[1];
}
__device__ inline float xrow16_f32(float v) { return __uint_as_float(xrow16_u32(__float_as_uint(v))); }
__device__ inline float xrow32_f32(float v) { return __uint_as_float(xrow32_u32(__float_as_uint(v))); }

// Combine across the four 16-lane rows only (lanes l, l^16, l^32, l^48).
__device__ inline float xrow_max(float v) {
  v = fmaxf(v, xrow16_f32(v));
  return fmaxf(v, xrow32_f32(v));
}
__device__ inline float xrow_sum(float v) {
  v += xrow16_f32(v);
  return v + xrow32_f32(v);
}

__device__ inline float wave_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return xrow_sum(v);
}

__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return xrow_max(v);
}

__device__ inline int wave_min_i32(int v) {
  v = min(v, static_cast<int>(dpp_u32<kDppXor1>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(dpp_u32<kDppXor2>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(dpp_u32<kDppHalfMirror>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(dpp_u32<kDppMirror>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(xrow16_u32(static_cast<uint32_t>(v))));
  return min(v, static_cast<int>(xrow32_u32(static_cast<uint32_t>(v))));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dg
