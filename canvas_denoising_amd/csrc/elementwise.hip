// Row-wise and elementwise kernels of the denoising step: token-embedding
// gather (+ the self-conditioning vector), RMSNorm, the tempered
// probabilities fed to self-conditioning, the embedding transpose and the
// packing of row-major expert matrices into their fragment-tiled layout.
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "mfma.h"
#include "prof.h"
#include "tiles.h"

namespace dg {

constexpr int kRowThreads = 256;

__device__ inline float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float t = sh[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) t += sh[w];
  __syncthreads();
  return t;
}

// x[m] = E[ids[m]] (+ sc[m]); fp32 residual stream. E is stored fragment-tiled in groups of
// kVocabGroup 16-row blocks (tiles.h): every 8 consecutive elements of a row are contiguous, so a
// thread gathers 8 at a time. Ids outside [0, V) are out of contract; they are clamped so that a
// bad id cannot read outside the table.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void embed_kernel(const T* __restrict__ emb, const int32_t* __restrict__ ids,
                                                             const float* __restrict__ sc, float* __restrict__ x,
                                                             int D, int V) {
  const int m = blockIdx.x;
  const int id = min(max(ids[m], 0), V - 1);
  for (int c = threadIdx.x; c < D / 8; c += kRowThreads) {
    const T* e = emb + tiled_index(id, 8 * c, 0, D, kVocabGroup, 1);
    float* xr = x + static_cast<int64_t>(m) * D + 8 * c;
    const float* sr = sc ? sc + static_cast<int64_t>(m) * D + 8 * c : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) xr[j] = to_f32<T>(e[j]) + (sr ? sr[j] : 0.f);
  }
}

// h = x / sqrt(mean(x^2) + eps) (unit gain); one workgroup per row, fixed summation order
template <typename T>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const float* __restrict__ x, T* __restrict__ h, int D,
                                                               float eps) {
  __shared__ float sh[kRowThreads / 64];
  const int m = blockIdx.x;
  const float* xr = x + static_cast<int64_t>(m) * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += kRowThreads) ss = fmaf(xr[i], xr[i], ss);
  ss = block_sum(ss, sh);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  T* hr = h + static_cast<int64_t>(m) * D;
  for (int i = threadIdx.x; i < D; i += kRowThreads) hr[i] = from_f32<T>(xr[i] * rs);
}

// Same, one wave per row with the row held in registers (D % 4 == 0, D <= 256 NV): one read of x,
// float4 loads, a fixed-order sum (per lane over its float4s, then the wave butterfly).
template <typename T, int NV>
__global__ __launch_bounds__(256) void rmsnorm_wave_kernel(const float* __restrict__ x, T* __restrict__ h, int M,
                                                           int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int n4 = D / 4;
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<int64_t>(m) * D);
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  T* hr = h + static_cast<int64_t>(m) * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < n4) {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(hr + 4 * c) =
            make_uint2(pack_bf16x2(v[i].x * rs, v[i].y * rs), pack_bf16x2(v[i].z * rs, v[i].w * rs));
      } else {
        *reinterpret_cast<float4*>(hr + 4 * c) = make_float4(v[i].x * rs, v[i].y * rs, v[i].z * rs, v[i].w * rs);
      }
    }
  }
}

// Residual update fused with the next RMSNorm, one workgroup per row, the row in registers
// (thread t holds float4 columns t, t + 256, ...; D % 4 == 0, D <= 1024 NV):
//   x[m] += sum_z part[z][m]                                  (z = 0 .. splits-1, in order)
//   x[m] += y[m] + sum_j slot_out[slot_of[m k + j]]           (when y != null; j in order; y[m] is
//                                                              the in-order sum of y_planes planes)
//   h[m]  = x[m] / sqrt(mean(x[m]^2) + eps)                   (fixed-order block sum)
// The first line folds the split-K partials of a GEMM whose epilogue adds into x; the second is the
// MoE combine (shared expert, then the token's gated routed outputs).
template <typename T, int NV>
__global__ __launch_bounds__(256) void residual_norm_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                            int splits, const float* __restrict__ y, int y_planes,
                                                            const float* __restrict__ slot_out,
                                                            const int32_t* __restrict__ slot_of, int k,
                                                            T* __restrict__ h, int M, int D, float eps) {
  __shared__ float sh[4];
  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const int n4 = D / 4;
  const int64_t plane = static_cast<int64_t>(M) * n4;  // float4s per partial
  float4* xr = reinterpret_cast<float4*>(x + static_cast<int64_t>(m) * D);
  const float4* p4 = reinterpret_cast<const float4*>(part);
  const float4* y4 = reinterpret_cast<const float4*>(y);
  const float4* s4 = reinterpret_cast<const float4*>(slot_out);
  constexpr int B = 8;  // gathered rows whose loads are issued together
  auto add4 = [](float4& t, const float4& u) { t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w; };
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + 256 * i;
    v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Gathered loads are unconditional (indices clamped into range, surplus values never added), so a
  // batch of B rows is in flight at once instead of issued one by one behind uniform branches.
  if (splits > 0) {  // t = part[0] + part[1] + ... (in order), x += t
    float4 t[NV];
    for (int z0 = 0; z0 < splits; z0 += B) {
      float4 u[NV][B];
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const int c = min(tid + 256 * i, n4 - 1);
          u[i][q] = p4[min(z0 + q, splits - 1) * plane + static_cast<int64_t>(m) * n4 + c];
        }
      // surplus values are replaced by zeros rather than skipped: a skipped value would let the
      // compiler sink its load behind a branch
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const float4 w = z0 + q < splits ? u[i][q] : make_float4(0.f, 0.f, 0.f, 0.f);
          if (z0 + q == 0) t[i] = w;
          else add4(t[i], w);
        }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (tid + 256 * i < n4) add4(v[i], t[i]);  // lanes past the row keep v = 0
  }
  if (y4) {  // t = y + slot_out[slot 0] + slot_out[slot 1] + ... (in order), x += t
    float4 t[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = tid + 256 * i;
      t[i] = c < n4 ? y4[static_cast<int64_t>(m) * n4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int p = 1; p < y_planes; ++p)  // y given as split partials: y = y[0] + y[1] + ... (in order)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = tid + 256 * i;
        if (c < n4) add4(t[i], y4[p * plane + static_cast<int64_t>(m) * n4 + c]);
      }
    for (int j0 = 0; j0 < k; j0 += B) {
      int sl[B];
#pragma unroll
      for (int q = 0; q < B; ++q) sl[q] = slot_of[m * k + min(j0 + q, k - 1)];
      float4 u[NV][B];
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const int c = min(tid + 256 * i, n4 - 1);
          u[i][q] = s4[static_cast<int64_t>(sl[q]) * n4 + c];
        }
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < B; ++q) add4(t[i], j0 + q < k ? u[i][q] : make_float4(0.f, 0.f, 0.f, 0.f));
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (tid + 256 * i < n4) add4(v[i], t[i]);  // lanes past the row keep v = 0
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + 256 * i;
    if (c < n4 && (splits > 0 || y4)) xr[c] = v[i];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) sh[tid >> 6] = ss;
  __syncthreads();
  ss = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  T* hr = h + static_cast<int64_t>(m) * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + 256 * i;
    if (c < n4) {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(hr + 4 * c) =
            make_uint2(pack_bf16x2(v[i].x * rs, v[i].y * rs), pack_bf16x2(v[i].z * rs, v[i].w * rs));
      } else {
        *reinterpret_cast<float4*>(hr + 4 * c) = make_float4(v[i].x * rs, v[i].y * rs, v[i].z * rs, v[i].w * rs);
      }
    }
  }
}

// P[m][v] = exp((l[m][v] - max_m) / T - lnZ_m): the sampler's tempered distribution,
// rebuilt from its row statistics (max raw logit, ln of the tempered partition sum)
// out[c][r] = in[r][c]; 64 x 64 tiles through LDS. `in` ([R x C]) is fragment-tiled with groups of gr
// 16-row blocks (tiles.h) when gr > 0, row-major otherwise; likewise `out` ([C x R]) with gr_out.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t R, int64_t C, int gr,
                                                        int gr_out, T* __restrict__ out) {
  __shared__ T tile[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = in[gr > 0 ? tiled_index(r, c, 0, C, gr, 1) : r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (r < R && c < C) out[gr_out > 0 ? tiled_index(c, r, 0, R, gr_out, 1) : c * R + r] = tile[tx][i];
  }
}

__global__ void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------------------- host
static int grid_for(int64_t n, int per = 256) {
  return static_cast<int>(std::min<int64_t>(std::max<int64_t>((n + per - 1) / per, 1), 8192));
}

int embed(const void* emb, const int32_t* ids, const float* sc, float* x, int M, int D, int V, int dtype,
          hipStream_t s) {
  ProfScope ps("embed", s);
  if (dtype == DG_BF16)
    embed_kernel<bf16_t><<<M, kRowThreads, 0, s>>>(static_cast<const bf16_t*>(emb), ids, sc, x, D, V);
  else
    embed_kernel<float><<<M, kRowThreads, 0, s>>>(static_cast<const float*>(emb), ids, sc, x, D, V);
  DG_LAUNCH_CHECK("embed_kernel");
  return DG_OK;
}

int rmsnorm(const float* x, void* h, int M, int D, float eps, int dtype, hipStream_t s) {
  ProfScope ps("rmsnorm", s);
  constexpr int kNV = 12;  // float4 per lane: rows up to 3072 wide take the one-wave kernel
  if (D % 4 == 0 && D <= 256 * kNV) {
    const int grid = (M + 3) / 4;
    if (dtype == DG_BF16)
      rmsnorm_wave_kernel<bf16_t, kNV><<<grid, 256, 0, s>>>(x, static_cast<bf16_t*>(h), M, D, eps);
    else
      rmsnorm_wave_kernel<float, kNV><<<grid, 256, 0, s>>>(x, static_cast<float*>(h), M, D, eps);
  } else if (dtype == DG_BF16) {
    rmsnorm_kernel<bf16_t><<<M, kRowThreads, 0, s>>>(x, static_cast<bf16_t*>(h), D, eps);
  } else {
    rmsnorm_kernel<float><<<M, kRowThreads, 0, s>>>(x, static_cast<float*>(h), D, eps);
  }
  DG_LAUNCH_CHECK("rmsnorm_kernel");
  return DG_OK;
}

int residual_norm(float* x, const float* part, int splits, const float* y, const float* slot_out,
                  const int32_t* slot_of, int k, void* h, int M, int D, float eps, int dtype, hipStream_t s,
                  const char* name, int y_planes) {
  if (y_planes < 1) return fail(DG_ERR_INVALID, "residual_norm: y_planes must be >= 1");
  constexpr int kNV = 3;
  if (D % 4 != 0 || D > 1024 * kNV || k > 16)
    return fail(DG_ERR_UNSUPPORTED, "residual_norm: d_model must be <= 3072 and a multiple of 4, top_k <= 16");
  ProfScope ps(name, s);
  if (dtype == DG_BF16)
    residual_norm_kernel<bf16_t, kNV><<<M, 256, 0, s>>>(x, part, splits, y, y_planes, slot_out, slot_of, k,
                                                       static_cast<bf16_t*>(h), M, D, eps);
  else
    residual_norm_kernel<float, kNV><<<M, 256, 0, s>>>(x, part, splits, y, y_planes, slot_out, slot_of, k,
                                                      static_cast<float*>(h), M, D, eps);
  DG_LAUNCH_CHECK("residual_norm_kernel");
  return DG_OK;
}

// *p = v on `s` (a one-thread kernel: a value the host decides for device code that reads it later,
// also from a captured graph, without a host-to-device copy)
__global__ void store_i32_kernel(int32_t* p, int32_t v) { *p = v; }
__global__ void store_f32_kernel(float* p, float v) { *p = v; }

int store_i32(int32_t* p, int32_t v, hipStream_t s) {
  store_i32_kernel<<<1, 1, 0, s>>>(p, v);
  DG_LAUNCH_CHECK("store_i32_kernel");
  return DG_OK;
}

int store_f32(float* p, float v, hipStream_t s) {
  store_f32_kernel<<<1, 1, 0, s>>>(p, v);
  DG_LAUNCH_CHECK("store_f32_kernel");
  return DG_OK;
}

int transpose(const void* in, int64_t R, int64_t C, int gr, int gr_out, void* out, int dtype, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((R + 63) / 64));
  if (grid.y > 65535) return fail(DG_ERR_UNSUPPORTED, "transpose: too many rows");
  if (dtype == DG_BF16)
    transpose_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(in), R, C, gr, gr_out,
                                                  static_cast<bf16_t*>(out));
  else
    transpose_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(in), R, C, gr, gr_out,
                                                 static_cast<float*>(out));
  DG_LAUNCH_CHECK("transpose_kernel");
  return DG_OK;
}

// dst[tiled_index(r, k)] = src[r * K + k] for one matrix of a tile group (tiles.h)
template <typename T>
__global__ void pack_tiled_kernel(const T* __restrict__ src, int64_t R, int64_t K, int which, int gr, int gw,
                                  T* __restrict__ dst) {
  const int64_t n = R * K;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / K, k = i - r * K;
    dst[tiled_index(r, k, which, K, gr, gw)] = src[i];
  }
}

int pack_tiled(const void* src, int64_t R, int64_t K, int which, int gr, int gw, void* dst, int dtype,
               hipStream_t s) {
  if (R % (16 * gr) != 0 || K % 32 != 0 || which < 0 || which >= gw)
    return fail(DG_ERR_INVALID, "pack_tiled: shape does not tile");
  const int64_t n = R * K;
  if (n == 0) return DG_OK;
  if (dtype == DG_BF16)
    pack_tiled_kernel<bf16_t><<<grid_for(n), 256, 0, s>>>(static_cast<const bf16_t*>(src), R, K, which, gr, gw,
                                                          static_cast<bf16_t*>(dst));
  else
    pack_tiled_kernel<float><<<grid_for(n), 256, 0, s>>>(static_cast<const float*>(src), R, K, which, gr, gw,
                                                         static_cast<float*>(dst));
  DG_LAUNCH_CHECK("pack_tiled_kernel");
  return DG_OK;
}

int zero_fill(void* p, size_t bytes, hipStream_t s) {
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(DG_ERR_INVALID, "zero_fill alignment");
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return DG_OK;
  zero_kernel<<<grid_for(n16), 256, 0, s>>>(static_cast<uint4*>(p), n16);
  DG_LAUNCH_CHECK("zero_kernel");
  return DG_OK;
}

}  // namespace dg

namespace dg {

// ------------------------------------------------------------ rotary positions
// Rotary position embedding (optional; the model's reading: the Gemma family's "rotate half" form):
// for j < hd / 2 the pair (x_j, x_{j + hd/2}) of every query and key head at cache position p is
// turned by the angle p * theta^(-2j / hd). cos and sin of every (position, j) are tabulated once,
// in double precision and rounded to float, so the rotation itself is a few multiplies.

// table[p][j] = (cos, sin) of p * theta^(-2j/hd), p < n_pos, j < hd / 2
__global__ void rope_table_kernel(double theta, int hd, int64_t n_pos, float2* __restrict__ table) {
  const int half = hd / 2;
  const int64_t n = n_pos * half;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int64_t p = e / half;
    const int j = static_cast<int>(e - p * half);
    const double a = static_cast<double>(p) * pow(theta, -2.0 * j / hd);
    table[e] = make_float2(static_cast<float>(cos(a)), static_cast<float>(sin(a)));
  }
}

// One thread per (row, head, pair): query heads of q (row-major [M][Hq * hd], ld ldq; skipped when q
// is null) and key heads of the cache rows at positions pos0 .. pos0 + M - 1 ([Hkv][cap][hd], head
// stride kv_stride), rotated in place in fp32 and rounded back to T.
template <typename T>
__global__ void rope_kernel(T* __restrict__ q, int64_t ldq, T* __restrict__ kc, int64_t kv_stride, int pos0,
                            const int* __restrict__ pos_dev, int M, int Hq, int Hkv, int hd,
                            const float2* __restrict__ table) {
  const int half = hd / 2;
  const int H = (q ? Hq : 0) + Hkv;
  const int64_t n = static_cast<int64_t>(M) * H * half;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int j = static_cast<int>(e % half);
  const int64_t rh = e / half;
  const int head = static_cast<int>(rh % H);
  const int row = static_cast<int>(rh / H);
  const int pos = (pos_dev ? *pos_dev : pos0) + row;
  T* x;
  if (q && head < Hq) x = q + static_cast<int64_t>(row) * ldq + static_cast<int64_t>(head) * hd;
  else x = kc + static_cast<int64_t>(head - (q ? Hq : 0)) * kv_stride + static_cast<int64_t>(pos) * hd;
  const float2 cs = table[static_cast<int64_t>(pos) * half + j];
  const float a = to_f32<T>(x[j]), b = to_f32<T>(x[j + half]);
  x[j] = from_f32<T>(a * cs.x - b * cs.y);
  x[j + half] = from_f32<T>(b * cs.x + a * cs.y);
}

int rope_table(double theta, int hd, int64_t n_pos, float2* table, hipStream_t s) {
  const int64_t n = n_pos * (hd / 2);
  if (n == 0) return DG_OK;
  rope_table_kernel<<<grid_for(n), 256, 0, s>>>(theta, hd, n_pos, table);
  DG_LAUNCH_CHECK("rope_table_kernel");
  return DG_OK;
}

int rope_apply(void* q, int64_t ldq, void* kc, int64_t kv_stride, int pos0, const int* pos_dev, int M, int Hq,
               int Hkv, int hd, const float2* table, int dtype, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(M) * ((q ? Hq : 0) + Hkv) * (hd / 2);
  if (n == 0) return DG_OK;
  ProfScope ps("rope", s);
  const unsigned grid = static_cast<unsigned>((n + 255) / 256);
  if (dtype == DG_BF16)
    rope_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<bf16_t*>(q), ldq, static_cast<bf16_t*>(kc), kv_stride, pos0,
                                             pos_dev, M, Hq, Hkv, hd, table);
  else
    rope_kernel<float><<<grid, 256, 0, s>>>(static_cast<float*>(q), ldq, static_cast<float*>(kc), kv_stride, pos0,
                                            pos_dev, M, Hq, Hkv, hd, table);
  DG_LAUNCH_CHECK("rope_kernel");
  return DG_OK;
}

}  // namespace dg
