// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11) and the uniform token draw used for the canvas
// initialisation and the re-noise of rejected positions ([P3] "Masked
// Diffusion vs Uniform State Diffusion": noise is a random token from the
// whole vocabulary; [P4] "How Uniform State Diffusion works": x ~ Uniform(V)).
//
// Key = (seed low word, seed high word); counter = (position, step, block,
// purpose) with purpose 0 for the initial canvas and 1 for re-noise; the draw
// takes output word 0 and maps it to floor(r * vocab / 2^32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// purpose 2: categorical sampling; token v uses purpose word 2 + 4 (v / 4) and output word v % 4
enum : uint32_t { kPurposeInit = 0, kPurposeRenoise = 1, kPurposeGumbel = 2 };

struct PhiloxOut { uint32_t w0, w1, w2, w3; };

__host__ __device__ inline void mulhilo32(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  const uint64_t p = static_cast<uint64_t>(a) * static_cast<uint64_t>(b);
  hi = static_cast<uint32_t>(p >> 32);
  lo = static_cast<uint32_t>(p);
}

__host__ __device__ inline PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                   uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint32_t hA, lA, hB, lB;
    mulhilo32(kMulA, c0, hA, lA);
    mulhilo32(kMulB, c2, hB, lB);
    const uint32_t n0 = hB ^ c1 ^ k0;
    const uint32_t n2 = hA ^ c3 ^ k1;
    c0 = n0; c1 = lB; c2 = n2; c3 = lA;
    k0 += kWeylA; k1 += kWeylB;
  }
  return {c0, c1, c2, c3};
}

__host__ __device__ inline int32_t draw_token(uint64_t seed, uint32_t pos, uint32_t step, uint32_t block,
                                              uint32_t purpose, uint32_t vocab) {
  const PhiloxOut o = philox4x32_10(pos, step, block, purpose, static_cast<uint32_t>(seed),
                                    static_cast<uint32_t>(seed >> 32));
  return static_cast<int32_t>((static_cast<uint64_t>(o.w0) * vocab) >> 32);
}

}  // namespace dg
