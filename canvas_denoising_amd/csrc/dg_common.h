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

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ------------------------------------------------------ wave64 reductions
template <typename T>
__device__ inline T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, 64); }

// Combine a value across the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48) with the
// gfx950 row swaps: v_permlane16_swap / v_permlane32_swap given the same register twice return, in
// one of their two results, the value of the partner row, so op(r0, r1) combines each pair (and,
// op being commutative, every lane of the pair gets the same bits). VALU only, no LDS round trip.
__device__ inline float xrow_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float xrow_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dg
