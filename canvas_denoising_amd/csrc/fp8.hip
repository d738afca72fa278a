// FP8 (OCP E4M3) storage of the routed experts' weights: an opt-in mode that
// halves the bytes the expert kernels stream. [P2] "24GB GPU: practical
// adoption and running conditions" lists quantised GGUF builds of the model
// (the 8-bit one at about half the bf16 footprint) and [P1] "Summary" points
// local runs at them; the storage here is this library's own, fitted to
// gfx950's FP8 conversions: E4M3 without infinities (bias 7, 3 fraction
// bits, subnormals in units of 2^-9, largest finite 448), one float32 scale
// per output row of each matrix:
// s = max|w| / 448 (1 for an all-zero row), code = E4M3(w / s) rounded to
// nearest-even and saturated at 448; the model computes with code * s.
//
// One wave per 16-row block of one matrix reads the block's bf16 tiles
// twice (row maxima, then codes) and writes the codes in the paired-tile
// order of tiles.h plus the 16 scales. Division is the correctly rounded
// float32 one, so codes and scales are a function of the weights alone.
#include "dg_common.h"
#include "prof.h"
#include "tiles.h"

namespace dg {

// E4M3 code of a float32 value: nearest, ties to an even fraction, |q| beyond 448's rounding range
// (464 is the midpoint to the next step, 480, which E4M3 spends on NaN) saturates to 448.
__device__ inline uint32_t e4m3_code(float q) {
  const uint32_t bits = __float_as_uint(q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  const float a = __uint_as_float(abits);
  uint32_t mag;
  if (a >= 464.f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal units of 2^-9 (8 units is the first normal code)
    mag = static_cast<uint32_t>(rintf(a * 512.f));
  } else {  // keep 3 of the 23 fraction bits, nearest-even; a carry moves to the next exponent
    int e = static_cast<int>(abits >> 23) - 127;
    uint32_t m = (abits >> 20) & 7u;
    const uint32_t rem = abits & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) { m = 0u; ++e; }
    mag = min((static_cast<uint32_t>(e + 7) << 3) | m, 0x7Eu);
  }
  return sign | mag;
}

// Grid: ceil(E * gw * R / 16 / 4) workgroups of 4 waves; wave w quantizes 16-row block rb of
// matrix `which` of expert e. src: bf16 tiles (tiles.h order, group width gr, gw matrices, K columns)
// per expert src_stride elements apart; codes: paired fp8 tiles per expert code_stride bytes apart;
// scales: [E][gw][R] float32.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const bf16_t* __restrict__ src, int64_t src_stride,
                                                           uint8_t* __restrict__ codes, int64_t code_stride,
                                                           float* __restrict__ scales, int E, int R, int K, int gr,
                                                           int gw) {
  const int lane = threadIdx.x & 63;
  const int RB = R / 16;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= static_cast<int64_t>(E) * gw * RB) return;
  const int e = static_cast<int>(w / (gw * RB));
  const int rem = static_cast<int>(w % (gw * RB));
  const int which = rem / RB, rb = rem % RB;
  const int G = gr * gw, KT = K / 32;
  const int group = rb / gr, g = which * gr + rb % gr;
  const bf16_t* s0 = src + e * src_stride + (static_cast<int64_t>(group) * KT * G + g) * kTileElems + lane * 8;
  float mx = 0.f;
  for (int kt = 0; kt < KT; ++kt) {
    const uint4 v = *reinterpret_cast<const uint4*>(s0 + static_cast<int64_t>(kt) * G * kTileElems);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(fabsf(bf16lo(u[j])), fabsf(bf16hi(u[j]))));
  }
  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same row
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float s = mx > 0.f ? __fdiv_rn(mx, 448.f) : 1.f;
  if (lane < 16) scales[(static_cast<int64_t>(e) * gw + which) * R + rb * 16 + lane] = s;
  uint8_t* c0 = codes + e * code_stride + (static_cast<int64_t>(group) * (KT / 2) * G + g) * 1024 + lane * 16;
  for (int kt = 0; kt < KT; ++kt) {
    const uint4 v = *reinterpret_cast<const uint4*>(s0 + static_cast<int64_t>(kt) * G * kTileElems);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = e4m3_code(__fdiv_rn(bf16lo(u[j]), s));
      const uint32_t hi = e4m3_code(__fdiv_rn(bf16hi(u[j]), s));
      out[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
    }
    *reinterpret_cast<uint2*>(c0 + static_cast<int64_t>(kt >> 1) * G * 1024 + (kt & 1) * 8) = make_uint2(out[0], out[1]);
  }
}

int quantize_fp8(const void* src, int64_t src_stride, void* codes, int64_t code_stride, float* scales, int E, int R,
                 int K, int gr, int gw, hipStream_t s) {
  if (R % (16 * gr) != 0 || K % 64 != 0)
    return fail(DG_ERR_UNSUPPORTED, "FP8 experts: rows must fill whole tile groups and K must be a multiple of 64");
  const int64_t waves = static_cast<int64_t>(E) * gw * (R / 16);
  if (waves == 0) return DG_OK;
  ProfScope ps("quantize_fp8", s);
  quantize_fp8_kernel<<<static_cast<unsigned>((waves + 3) / 4), 256, 0, s>>>(
      static_cast<const bf16_t*>(src), src_stride, static_cast<uint8_t*>(codes), code_stride, scales, E, R, K, gr, gw);
  DG_LAUNCH_CHECK("quantize_fp8_kernel");
  return DG_OK;
}

}  // namespace dg
