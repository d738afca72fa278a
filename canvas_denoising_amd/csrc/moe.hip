// Sparse MoE FFN: router top-k, token permutation and weight-streaming grouped
// expert GEMMs ([P4] "Gemma-based MoE backbone", table: 8 of 128 experts
// active plus 1 shared; [P3] "Encoder-denoiser design": the denoiser is the
// Gemma 4 26B-A4B MoE backbone).
//
// Routing (one workgroup): per row, softmax over the E router logits and the
// top-k chosen on the logits themselves (largest first, lowest index on
// ties); the gate is the selected softmax probability. Every (token, expert)
// pair sets a bit in a per-expert token mask in LDS; popcounts give expert
// sizes, an exclusive scan gives offsets, and a token's rank inside its
// expert is the popcount of the mask bits below it. The slot order is
// therefore expert-major and token-ascending whatever the thread timing.
//
// Expert GEMMs: with a 256-token canvas an expert sees about 16 tokens, so
// the work is a stream of expert weights (arithmetic intensity ~16 flop/B).
// Each wave owns 16 output features of one expert and streams their weight
// rows straight from HBM into MFMA B fragments (16-byte loads, 4 k-steps
// of 32 in flight), while the expert's gathered token rows (A fragments) come
// from L2. Up to 64 tokens are kept in accumulators per pass; an expert with
// more tokens takes further passes. No LDS, no barriers: waves are independent.
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "mfma.h"
#include "prof.h"

namespace dg {

constexpr int kRouteThreads = 1024;
constexpr int kMaxTokens = 256;     // rows per routing call
constexpr int kMaskWords = kMaxTokens / 32;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, int M, int E, int k, int renorm,
    int32_t* __restrict__ sel, float* __restrict__ gate, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot_of, float* __restrict__ slot_gate) {
  __shared__ uint32_t mask[256 * kMaskWords];  // E <= 256
  __shared__ int32_t offs[257];
  __shared__ int32_t lsel[kMaxTokens * 16];     // k <= 16
  __shared__ float lgate[kMaxTokens * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < E * kMaskWords; i += kRouteThreads) mask[i] = 0u;
  __syncthreads();

  constexpr int kPer = 4;  // values per lane (E <= 256)
  for (int row = wave; row < M; row += kRouteThreads / 64) {
    float v[kPer];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? logits[static_cast<int64_t>(row) * E + e] : -INFINITY;
      mx = fmaxf(mx, v[i]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) sum += (lane + 64 * i < E) ? expf(v[i] - mx) : 0.f;
    sum = wave_sum(sum);
    float gsum = 0.f;
    float gsel[16];
    int esel[16];
    for (int j = 0; j < k; ++j) {
      // wave argmax: largest value, lowest expert index on ties
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = shfl_xor(bv, m);
        const int oe = shfl_xor(be, m);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i == be) v[i] = -INFINITY;
      const float g = expf(bv - mx) / sum;
      gsel[j] = g;
      esel[j] = be;
      gsum += g;
    }
    if (lane == 0) {
      for (int j = 0; j < k; ++j) {
        const float g = renorm ? gsel[j] / gsum : gsel[j];
        sel[row * k + j] = esel[j];
        gate[row * k + j] = g;
        lsel[row * k + j] = esel[j];
        lgate[row * k + j] = g;
        atomicOr(&mask[esel[j] * kMaskWords + (row >> 5)], 1u << (row & 31));
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of expert sizes (E <= 256: 4 per lane)
    int cnt[4];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int c = 0;
      if (e < E)
        for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e * kMaskWords + w]);
      cnt[i] = c;
      tot += c;
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    int run = incl - tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) offs[e] = run;
      run += cnt[i];
    }
    if (lane == 63) offs[E] = incl;
  }
  __syncthreads();
  for (int i = tid; i <= E; i += kRouteThreads) offsets[i] = offs[i];
  for (int p = tid; p < M * k; p += kRouteThreads) {
    const int row = p / k;
    const int e = lsel[p];
    int rank = 0;
    for (int w = 0; w < (row >> 5); ++w) rank += __popc(mask[e * kMaskWords + w]);
    rank += __popc(mask[e * kMaskWords + (row >> 5)] & ((1u << (row & 31)) - 1u));
    const int slot = offs[e] + rank;
    perm[slot] = row;
    slot_of[p] = slot;
    slot_gate[slot] = lgate[p];
  }
}

// ------------------------------------------------------------------ experts
constexpr int kExpWaves = 4;
constexpr int kMT = 4;       // 16-token tiles held per pass (64 tokens)
constexpr int kKC = 4;       // k-steps of 32 per loaded chunk

// act[slot][j] = GeLU(h W_gate[e]^T)_j * (h W_up[e]^T)_j  (GATED) or GeLU(h W_up[e]^T)_j
// for the slots of expert e. Grid: (ceil(F / 64), E); wave w owns features j0 .. j0+15.
template <typename T, bool GATED>
__global__ __launch_bounds__(256) void expert_gateup_kernel(
    const T* __restrict__ h, int64_t ldh, const T* __restrict__ w_gu, int64_t expert_stride, int F, int D,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, T* __restrict__ act) {
  using Fr = Frag<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int j0 = (blockIdx.x * kExpWaves + wave) * 16;
  if (j0 >= F) return;
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const T* wbase = w_gu + static_cast<int64_t>(e) * expert_stride;
  const T* wu = wbase + static_cast<int64_t>(GATED ? F + j0 + fr : j0 + fr) * D + fk;
  const T* wg = wbase + static_cast<int64_t>(j0 + fr) * D + fk;

  for (int p0 = 0; p0 < cnt; p0 += kMT * 16) {
    const int ntile = min(kMT, (cnt - p0 + 15) / 16);
    const T* arow[kMT];
    bool aok[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      const int s = p0 + t * 16 + fr;
      aok[t] = t < ntile && s < cnt;
      arow[t] = h + static_cast<int64_t>(aok[t] ? perm[beg + s] : 0) * ldh + fk;
    }
    f32x4_t accg[kMT], accu[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) { accg[t] = f32x4_t{0, 0, 0, 0}; accu[t] = f32x4_t{0, 0, 0, 0}; }
    for (int k0 = 0; k0 < D; k0 += 32 * kKC) {
      typename Fr::type bu[kKC], bg[kKC];
#pragma unroll
      for (int c = 0; c < kKC; ++c) {
        if (k0 + c * 32 < D) {
          bu[c] = Fr::load(wu + k0 + c * 32);
          if (GATED) bg[c] = Fr::load(wg + k0 + c * 32);
        }
      }
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        if (t < ntile) {
#pragma unroll
          for (int c = 0; c < kKC; ++c) {
            if (k0 + c * 32 < D) {
              const typename Fr::type a = aok[t] ? Fr::load(arow[t] + k0 + c * 32) : Fr::zero();
              accu[t] = Fr::mma(a, bu[c], accu[t]);
              if (GATED) accg[t] = Fr::mma(a, bg[c], accg[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      if (t < ntile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = p0 + t * 16 + (lane >> 4) * 4 + i;
          if (s < cnt) {
            const float v = GATED ? gelu_erf(accg[t][i]) * accu[t][i] : gelu_erf(accu[t][i]);
            act[static_cast<int64_t>(beg + s) * F + j0 + fr] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

// out[slot][n] = gate[slot] * sum_f act[slot][f] W_down[e][n][f]; grid (ceil(D / 64), E)
template <typename T>
__global__ __launch_bounds__(256) void expert_down_kernel(
    const T* __restrict__ act, const T* __restrict__ w_down, int64_t expert_stride, int F, int D,
    const int32_t* __restrict__ offsets, const float* __restrict__ slot_gate, float* __restrict__ out) {
  using Fr = Frag<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int n0 = (blockIdx.x * kExpWaves + wave) * 16;
  if (n0 >= D) return;
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const T* wrow = w_down + static_cast<int64_t>(e) * expert_stride + static_cast<int64_t>(n0 + fr) * F + fk;

  for (int p0 = 0; p0 < cnt; p0 += kMT * 16) {
    const int ntile = min(kMT, (cnt - p0 + 15) / 16);
    const T* arow[kMT];
    bool aok[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      const int s = p0 + t * 16 + fr;
      aok[t] = t < ntile && s < cnt;
      arow[t] = act + static_cast<int64_t>(beg + (aok[t] ? s : 0)) * F + fk;
    }
    f32x4_t acc[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) acc[t] = f32x4_t{0, 0, 0, 0};
    for (int k0 = 0; k0 < F; k0 += 32 * kKC) {
      typename Fr::type b[kKC];
#pragma unroll
      for (int c = 0; c < kKC; ++c)
        if (k0 + c * 32 < F) b[c] = Fr::load(wrow + k0 + c * 32);
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        if (t < ntile) {
#pragma unroll
          for (int c = 0; c < kKC; ++c) {
            if (k0 + c * 32 < F) {
              const typename Fr::type a = aok[t] ? Fr::load(arow[t] + k0 + c * 32) : Fr::zero();
              acc[t] = Fr::mma(a, b[c], acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      if (t < ntile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = p0 + t * 16 + (lane >> 4) * 4 + i;
          if (s < cnt) out[static_cast<int64_t>(beg + s) * D + n0 + fr] = slot_gate[beg + s] * acc[t][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------- host
int moe_route(const float* logits, int M, int E, int k, int renorm, int32_t* sel, float* gate, int32_t* offsets,
              int32_t* perm, int32_t* slot_of, float* slot_gate, hipStream_t s) {
  if (M > kMaxTokens || E > 256 || k > 16 || k > E) return fail(DG_ERR_UNSUPPORTED, "routing limits: M<=256, E<=256, k<=16");
  ProfScope ps("moe_route", s);
  route_kernel<<<1, kRouteThreads, 0, s>>>(logits, M, E, k, renorm, sel, gate, offsets, perm, slot_of, slot_gate);
  DG_LAUNCH_CHECK("route_kernel");
  return DG_OK;
}

int moe_experts(const void* h, int64_t ldh, const void* w_gu, const void* w_down, int E, int F, int D, int gated,
                const int32_t* offsets, const int32_t* perm, const float* slot_gate, void* act, float* out,
                int dtype, hipStream_t s) {
  if (F % 16 != 0 || D % 32 != 0) return fail(DG_ERR_UNSUPPORTED, "expert widths must be multiples of 16 / 32");
  const int64_t gu_stride = static_cast<int64_t>(gated ? 2 : 1) * F * D;
  const int64_t dn_stride = static_cast<int64_t>(D) * F;
  dim3 g1((F + 16 * kExpWaves - 1) / (16 * kExpWaves), E);
  dim3 g2((D + 16 * kExpWaves - 1) / (16 * kExpWaves), E);
  {
    ProfScope ps("expert_gateup", s);
    if (dtype == DG_BF16) {
      if (gated)
        expert_gateup_kernel<bf16_t, true><<<g1, 256, 0, s>>>(static_cast<const bf16_t*>(h), ldh,
            static_cast<const bf16_t*>(w_gu), gu_stride, F, D, offsets, perm, static_cast<bf16_t*>(act));
      else
        expert_gateup_kernel<bf16_t, false><<<g1, 256, 0, s>>>(static_cast<const bf16_t*>(h), ldh,
            static_cast<const bf16_t*>(w_gu), gu_stride, F, D, offsets, perm, static_cast<bf16_t*>(act));
    } else {
      if (gated)
        expert_gateup_kernel<float, true><<<g1, 256, 0, s>>>(static_cast<const float*>(h), ldh,
            static_cast<const float*>(w_gu), gu_stride, F, D, offsets, perm, static_cast<float*>(act));
      else
        expert_gateup_kernel<float, false><<<g1, 256, 0, s>>>(static_cast<const float*>(h), ldh,
            static_cast<const float*>(w_gu), gu_stride, F, D, offsets, perm, static_cast<float*>(act));
    }
  }
  DG_LAUNCH_CHECK("expert_gateup_kernel");
  {
    ProfScope ps("expert_down", s);
    if (dtype == DG_BF16)
      expert_down_kernel<bf16_t><<<g2, 256, 0, s>>>(static_cast<const bf16_t*>(act),
          static_cast<const bf16_t*>(w_down), dn_stride, F, D, offsets, slot_gate, out);
    else
      expert_down_kernel<float><<<g2, 256, 0, s>>>(static_cast<const float*>(act),
          static_cast<const float*>(w_down), dn_stride, F, D, offsets, slot_gate, out);
  }
  DG_LAUNCH_CHECK("expert_down_kernel");
  return DG_OK;
}

}  // namespace dg
