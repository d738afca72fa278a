// Seeded synthetic inputs on the device (random-init weights, prompts,
// planted-peak logits). No arithmetic of the denoising method lives here.
//
// Generator: hash64(seed, tid, i) = mix64(mix64(seed * G + tid) + (i + 1) * G)
// with the SplitMix64 finaliser mix64 (Steele, Lea and Flood, OOPSLA 2014)
// and G = 0x9E3779B97F4A7C15. A "normal" value is the Irwin-Hall sum of the
// hash's four 16-bit fields minus 131070, times float(sigma / sqrt((2^32 - 1) / 3))
// in one correctly rounded float multiply; bf16 rounds that to nearest-even.
// The background of the planted-peak logits sums the twelve fields of the
// hashes of indices 3 i, 3 i + 1 and 3 i + 2 (minus 393210, times
// float(sigma / sqrt(2^32 - 1))): tails to 6 sigma, so the largest of a row's
// 262144 values (about 4.2 sigma) competes with a planted peak about as a
// normal's would.
// A uniform id is ((hash >> 32) * V) >> 32. The host generator used by the
// tests computes the same bits.
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "prof.h"
#include "tiles.h"

// Keep every multiply and add separately rounded (no FMA contraction) so the
// values match the host generator bit for bit.
#pragma clang fp contract(off)

namespace dg {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTidLogits = 20, kTidPeak = 21;
constexpr uint32_t kPeakFractionNum = 3006477107u;  // floor(0.7 * 2^32)

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t tid) { return mix64(seed * kGolden + tid); }

__device__ inline float irwin_hall4(uint64_t h) {
  const int64_t s = static_cast<int64_t>(h & 0xFFFF) + static_cast<int64_t>((h >> 16) & 0xFFFF) +
                    static_cast<int64_t>((h >> 32) & 0xFFFF) + static_cast<int64_t>(h >> 48);
  return static_cast<float>(s - 131070);
}

__device__ inline int64_t fields_sum(uint64_t h) {
  return static_cast<int64_t>(h & 0xFFFF) + static_cast<int64_t>((h >> 16) & 0xFFFF) +
         static_cast<int64_t>((h >> 32) & 0xFFFF) + static_cast<int64_t>(h >> 48);
}

// twelve-field sum for element i of stream `key` (hash indices 3 i .. 3 i + 2)
__device__ inline float irwin_hall12(uint64_t key, int64_t i) {
  const uint64_t j = 3 * static_cast<uint64_t>(i);
  const int64_t s = fields_sum(mix64(key + (j + 1) * kGolden)) + fields_sum(mix64(key + (j + 2) * kGolden)) +
                    fields_sum(mix64(key + (j + 3) * kGolden));
  return static_cast<float>(s - 393210);
}

float normal12_scale(float sigma) {
  return static_cast<float>(static_cast<double>(sigma) / std::sqrt(65536.0 * 65536.0 - 1.0));
}

float normal_scale(float sigma) {
  const double sd4 = std::sqrt((65536.0 * 65536.0 - 1.0) / 3.0);
  return static_cast<float>(static_cast<double>(sigma) / sd4);
}

template <typename T>
__global__ void synth_normal_kernel(uint64_t key, int64_t n, float scale, T* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = irwin_hall4(mix64(key + static_cast<uint64_t>(i + 1) * kGolden)) * scale;
    if constexpr (sizeof(T) == 2) out[i] = f32_to_bf16(v);
    else out[i] = v;
  }
}

// Fill of a fragment-tiled tensor group (tiles.h): physical element p holds
// the value that stream keys[which] gives row-major element r * K + k of its
// matrix, i.e. the same values as synth_normal_kernel over each matrix.
template <typename T>
__global__ void synth_tiled_kernel(uint64_t key0, uint64_t key1, int64_t n, int64_t K, int gr, int gw, float scale,
                                   T* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < n; p += stride) {
    int which;
    int64_t r, k;
    tiled_coords(p, K, gr, gw, &which, &r, &k);
    const uint64_t key = which ? key1 : key0;
    const float v = irwin_hall4(mix64(key + static_cast<uint64_t>(r * K + k + 1) * kGolden)) * scale;
    if constexpr (sizeof(T) == 2) out[p] = f32_to_bf16(v);
    else out[p] = v;
  }
}

__global__ void synth_ids_kernel(uint64_t key, int64_t n, uint32_t vocab, int32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t h = mix64(key + static_cast<uint64_t>(i + 1) * kGolden);
    out[i] = static_cast<int32_t>(((h >> 32) * vocab) >> 32);
  }
}

__global__ void synth_logits_kernel(uint64_t key_bg, uint64_t key_pk, int rows, int64_t vocab, float scale,
                                    float peak, bf16_t* __restrict__ out) {
  const int64_t n = static_cast<int64_t>(rows) * vocab;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    float v = irwin_hall12(key_bg, i) * scale;
    const int64_t row = i / vocab, col = i - row * vocab;
    const uint64_t h = mix64(key_pk + static_cast<uint64_t>(row + 1) * kGolden);
    const bool planted = static_cast<uint32_t>(h) < kPeakFractionNum;
    const int64_t pc = static_cast<int64_t>(((h >> 32) * static_cast<uint64_t>(vocab)) >> 32);
    if (planted && col == pc) v = v + peak;
    out[i] = f32_to_bf16(v);
  }
}

static int grid_for(int64_t n) { return static_cast<int>(std::min<int64_t>(std::max<int64_t>(ceil_div(n, 256), 1), 65536)); }

// Calibration: a plain streaming read of n16 16-byte words, the ceiling a bandwidth-bound kernel of
// this library can aim at. Grid-stride, 4 nontemporal 16-byte loads in flight per thread per
// iteration; each thread folds its words with XOR and its workgroup writes one word to sink[block],
// so no load can be elided.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride), d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  ProfScope ps("stream_read", s);
  stream_read_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  DG_LAUNCH_CHECK("stream_read_kernel");
  return DG_OK;
}

int launch_synth_normal(uint64_t seed, uint64_t tid, int64_t n, float sigma, int dtype, void* out, hipStream_t s) {
  if (n == 0) return DG_OK;
  const uint64_t key = stream_key(seed, tid);
  const float scale = normal_scale(sigma);
  if (dtype == DG_BF16)
    synth_normal_kernel<bf16_t><<<grid_for(n), 256, 0, s>>>(key, n, scale, static_cast<bf16_t*>(out));
  else
    synth_normal_kernel<float><<<grid_for(n), 256, 0, s>>>(key, n, scale, static_cast<float*>(out));
  DG_LAUNCH_CHECK("synth_normal_kernel");
  return DG_OK;
}

// gw (1 or 2) matrices of R x K, streams tids[0 .. gw-1], stored tiled with gr row blocks per group
int launch_synth_tiled(uint64_t seed, const uint64_t* tids, int64_t R, int64_t K, int gr, int gw, float sigma,
                       int dtype, void* out, hipStream_t s) {
  const int64_t n = R * K * gw;
  if (n == 0) return DG_OK;
  const uint64_t k0 = stream_key(seed, tids[0]);
  const uint64_t k1 = gw > 1 ? stream_key(seed, tids[1]) : k0;
  const float scale = normal_scale(sigma);
  if (dtype == DG_BF16)
    synth_tiled_kernel<bf16_t><<<grid_for(n), 256, 0, s>>>(k0, k1, n, K, gr, gw, scale, static_cast<bf16_t*>(out));
  else
    synth_tiled_kernel<float><<<grid_for(n), 256, 0, s>>>(k0, k1, n, K, gr, gw, scale, static_cast<float*>(out));
  DG_LAUNCH_CHECK("synth_tiled_kernel");
  return DG_OK;
}

int launch_synth_ids(uint64_t seed, uint64_t tid, int64_t n, int vocab, int32_t* out, hipStream_t s) {
  if (n == 0) return DG_OK;
  synth_ids_kernel<<<grid_for(n), 256, 0, s>>>(stream_key(seed, tid), n, static_cast<uint32_t>(vocab), out);
  DG_LAUNCH_CHECK("synth_ids_kernel");
  return DG_OK;
}

int launch_synth_logits(uint64_t seed, int step, int rows, int vocab, float sigma, float peak, void* out,
                        hipStream_t s) {
  const int64_t n = static_cast<int64_t>(rows) * vocab;
  if (n == 0) return DG_OK;
  const uint64_t kb = stream_key(seed, kTidLogits + (static_cast<uint64_t>(step) << 8));
  const uint64_t kp = stream_key(seed, kTidPeak + (static_cast<uint64_t>(step) << 8));
  synth_logits_kernel<<<grid_for(n), 256, 0, s>>>(kb, kp, rows, vocab, normal12_scale(sigma), peak,
                                                  static_cast<bf16_t*>(out));
  DG_LAUNCH_CHECK("synth_logits_kernel");
  return DG_OK;
}

}  // namespace dg
