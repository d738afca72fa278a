// Sparse MoE FFN: router top-k, token permutation and weight-streaming grouped
// expert GEMMs ([P4] "Gemma-based MoE backbone", table: 8 of 128 experts
// active plus 1 shared; [P3] "Encoder-denoiser design": the denoiser is the
// Gemma 4 26B-A4B MoE backbone).
//
// Routing after the router product r = h W_r^T (a split-k GEMM whose
// partials are left unsummed), two kernels. (1) One wave per row: the
// partials summed in split order, softmax over the E logits, top-k on the
// logits themselves (largest first, lowest index on ties), the gate being
// the selected softmax probability. (2) One workgroup: every (token, expert)
// pair sets a bit in a per-expert token mask in LDS; popcounts give expert
// sizes, an exclusive scan gives offsets, and a token's rank inside its
// expert is the popcount of the mask bits below it. The slot order is
// therefore expert-major and token-ascending whatever the timing. The same
// kernel ranks the experts by token count (largest first, lower index on
// ties) for the expert kernels' block order.
//
// Expert GEMMs: with a 256-token canvas an expert sees about 16 tokens, so
// the work is a stream of expert weights (arithmetic intensity ~16 flop/B):
// HBM-bound, and with a loaded HBM latency of a few microseconds it is
// latency-bound unless many bytes are in flight, and DRAM-page-bound unless
// those bytes come in long contiguous runs. The weights are stored
// fragment-tiled (tiles.h): a workgroup owns one or two tile groups (gate/up:
// 32 features, gate and up; down: two groups of 64 output rows), each a
// contiguous stretch of memory, and its 4 waves split the k-tiles so that
// each stage of loads is one contiguous run per group with 1 KB per load
// instruction, straight into MFMA B fragments through a ring of register
// stages, together with the expert's gathered token rows (A fragments, from
// L2). The waves' partial sums meet in LDS at the end. Up to 64 tokens are
// held in accumulators per pass; an expert with more tokens takes further
// passes.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "dg_common.h"
#include "dma.h"
#include "mfma.h"
#include "prof.h"
#include "tiles.h"

namespace dg {

constexpr int kMaxTokens = 256;        // rows per routing call of a canvas
constexpr int kMaxTokensLarge = 4096;  // rows per routing call of a prefill chunk (E <= 128)
constexpr int kTileTokens = 128;       // token rows per workgroup of the token-tiled expert kernels

// keep the larger value, the lower expert index on ties (exact, so every lane agrees)
__device__ inline void argmax_step(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
}

// One wave routes one row of E <= 256 logits (lg, fp32): sel[0..k) the chosen experts in order,
// gate[0..k) their softmax probabilities (renormalised over the k when renorm).
__device__ inline void route_row(const float* lg, int E, int k, int renorm, int lane, int32_t* sel, float* gate) {
  constexpr int kPer = 4;  // E <= 256
  float v[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? lg[e] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) sum += (lane + 64 * i < E) ? expf(v[i] - mx) : 0.f;
  sum = wave_sum(sum);
  float my_gate = 0.f;
  int my_e = 0;
  float gsum = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
    }
    argmax_step(bv, be, dpp_f32<kDppXor1>(bv), static_cast<int>(dpp_u32<kDppXor1>(static_cast<uint32_t>(be))));
    argmax_step(bv, be, dpp_f32<kDppXor2>(bv), static_cast<int>(dpp_u32<kDppXor2>(static_cast<uint32_t>(be))));
    argmax_step(bv, be, dpp_f32<kDppHalfMirror>(bv),
                static_cast<int>(dpp_u32<kDppHalfMirror>(static_cast<uint32_t>(be))));
    argmax_step(bv, be, dpp_f32<kDppMirror>(bv), static_cast<int>(dpp_u32<kDppMirror>(static_cast<uint32_t>(be))));
    argmax_step(bv, be, xrow16_f32(bv), static_cast<int>(xrow16_u32(static_cast<uint32_t>(be))));
    argmax_step(bv, be, xrow32_f32(bv), static_cast<int>(xrow32_u32(static_cast<uint32_t>(be))));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i == be) v[i] = -INFINITY;
    const float g = expf(bv - mx) / sum;
    gsum += g;
    if (lane == j) { my_gate = g; my_e = be; }  // lane j keeps choice j
  }
  if (lane < k) {
    sel[lane] = my_e;
    gate[lane] = renorm ? my_gate / gsum : my_gate;
  }
}

// one workgroup of 1024 threads: expert sizes, offsets and the expert-major, token-ascending slot order.
// offsets holds E + 1 slot offsets followed by the E experts in order of decreasing token count
// (lower index first on ties).
// MW mask words per expert cover 32 MW rows (E <= min(256, 16384 / MW)). With `tiles`, also the list of the
// experts' 128-token tiles: tiles[0] = their number, tiles[1 + i] = e * 65536 + (tile within e),
// experts in order.
template <int MW>
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ sel,
                                                       const float* __restrict__ gate, int M, int E, int k,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ slot_of,
                                                       float* __restrict__ slot_gate, int32_t* __restrict__ tiles) {
  constexpr int kE = 16384 / MW < 256 ? 16384 / MW : 256;
  __shared__ uint32_t mask[kE * MW];
  __shared__ uint16_t below[kE * MW];  // tokens of expert e in the mask words before word w
  __shared__ int32_t offs[257];
  __shared__ int32_t toffs[257];
  __shared__ int32_t cnts[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < E * MW; i += 1024) mask[i] = 0u;
  // (token, choice) pairs in batches of 8 per thread whose loads are issued together (clamped
  // indices; surplus pairs are not used). The first batch's experts and gates stay in registers for
  // the slot scatter at the end (a canvas has at most 2048 pairs: one batch covers them all).
  const int np = M * k;
  constexpr int kPB = 8;
  int ev0[kPB];
  float gv0[kPB];
#pragma unroll
  for (int i = 0; i < kPB; ++i) {
    const int p = min(tid + 1024 * i, np - 1);
    ev0[i] = sel[p];
    gv0[i] = gate[p];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPB; ++i) {
    const int p = tid + 1024 * i, row = p / k;
    if (p < np) atomicOr(&mask[ev0[i] * MW + (row >> 5)], 1u << (row & 31));
  }
  for (int p0 = tid + 1024 * kPB; p0 < np; p0 += 1024 * kPB) {
    int ev[kPB];
#pragma unroll
    for (int i = 0; i < kPB; ++i) ev[i] = sel[min(p0 + 1024 * i, np - 1)];
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      const int p = p0 + 1024 * i, row = p / k;
      if (p < np) atomicOr(&mask[ev[i] * MW + (row >> 5)], 1u << (row & 31));
    }
  }
  __syncthreads();
  if (wave == 0) {
    int cnt[4];
    int tot = 0, ttot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int c = 0;
      if (e < E)
        for (int w = 0; w < MW; ++w) c += __popc(mask[e * MW + w]);
      cnt[i] = c;
      tot += c;
      ttot += (c + kTileTokens - 1) / kTileTokens;
    }
    int incl = tot, tincl = ttot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      const int to = __shfl_up(tincl, d, 64);
      if (lane >= d) { incl += o; tincl += to; }
    }
    int run = incl - tot, trun = tincl - ttot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) { offs[e] = run; toffs[e] = trun; cnts[e] = cnt[i]; }
      run += cnt[i];
      trun += (cnt[i] + kTileTokens - 1) / kTileTokens;
    }
    if (lane == 63) { offs[E] = incl; toffs[E] = tincl; }
  }
  // running popcounts of each expert's mask words, so a token's rank is one lookup and one popcount
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int w = 0; w < MW; ++w) {
      below[e * MW + w] = static_cast<uint16_t>(run);
      run += __popc(mask[e * MW + w]);
    }
  }
  __syncthreads();
  for (int i = tid; i <= E; i += 1024) offsets[i] = offs[i];
  // rank of expert e (most tokens first, lower index on ties): 8 threads per expert each count the
  // experts ahead of it in one eighth of the experts, summed across the 8 lanes
  constexpr int kSl = 8;
  const int per = (E + kSl - 1) / kSl;
  for (int base = 0; base < E * kSl; base += 1024) {
    const int t = base + tid, e = t / kSl, part = t % kSl;
    int r = 0;
    if (e < E) {
      const int c = cnts[e];
      const int f1 = min(E, (part + 1) * per);
      for (int f = part * per; f < f1; ++f) {
        const int cf = cnts[f];
        r += (cf > c || (cf == c && f < e)) ? 1 : 0;
      }
    }
    r += __shfl_xor(r, 1, 64);
    r += __shfl_xor(r, 2, 64);
    r += __shfl_xor(r, 4, 64);
    if (e < E && part == 0) offsets[E + 1 + r] = e;
  }
  if (tiles) {
    if (tid == 0) tiles[0] = toffs[E];
    for (int e = tid; e < E; e += 1024)
      for (int j = toffs[e]; j < toffs[e + 1]; ++j) tiles[1 + j] = e * 65536 + (j - toffs[e]);
  }
  auto scatter = [&](int p, int e, float gv) {
    const int row = p / k;
    const int rank = below[e * MW + (row >> 5)] + __popc(mask[e * MW + (row >> 5)] & ((1u << (row & 31)) - 1u));
    const int slot = offs[e] + rank;
    perm[slot] = row;
    slot_of[p] = slot;
    slot_gate[slot] = gv;
  };
#pragma unroll
  for (int i = 0; i < kPB; ++i) {
    const int p = tid + 1024 * i;
    if (p < np) scatter(p, ev0[i], gv0[i]);
  }
  for (int p0 = tid + 1024 * kPB; p0 < np; p0 += 1024 * kPB) {
    int ev[kPB];
    float gv[kPB];
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      const int p = min(p0 + 1024 * i, np - 1);
      ev[i] = sel[p];
      gv[i] = gate[p];
    }
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      const int p = p0 + 1024 * i;
      if (p < np) scatter(p, ev[i], gv[i]);
    }
  }
}

constexpr int kRouteSplits = 32;  // most split-k partials a routing call sums

// Grid ceil(M / W), W = kRouteWaves waves: wave w routes row W blockIdx.x + w. The logits are the sum of KS <= NS
// partials part[q * M * E + row * E + e] (KS = 1: part holds the logits), written to rlog. The NS
// loads of a column are unconditional (slots past KS re-read the last one and are not added), so
// they are all in flight together rather than issued one by one behind branches.
#ifndef DG_ROUTE_WAVES
#define DG_ROUTE_WAVES 2
#endif
constexpr int kRouteWaves = DG_ROUTE_WAVES;  // rows (one per wave) per workgroup

template <int NS>
__global__ __launch_bounds__(64 * kRouteWaves) void route_topk_kernel(const float* part, int M, int E, int k,
                                                                      int renorm, int KS, float* rlog,
                                                                      int32_t* __restrict__ sel,
                                                                      float* __restrict__ gate) {
  __shared__ float lg[kRouteWaves * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * kRouteWaves + wave;
  if (row >= M) return;
  const int64_t pstride = static_cast<int64_t>(M) * E;
  float* l = lg + wave * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (64 * i >= E) break;
    const int c = min(lane + 64 * i, E - 1);
    const float* pc = part + static_cast<int64_t>(row) * E + c;
    float v[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) v[q] = pc[min(q, KS - 1) * pstride];
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NS; ++q) sum += q < KS ? v[q] : 0.f;
    if (lane + 64 * i < E) {
      l[c] = sum;
      rlog[static_cast<int64_t>(row) * E + c] = sum;
    }
  }
  route_row(l, E, k, renorm, lane, sel + row * k, gate + row * k);
}

// ------------------------------------------------------------------ experts
#ifndef DG_EXP_KSP_GU
#define DG_EXP_KSP_GU 2
#endif
#ifndef DG_EXP_NS_GU
#define DG_EXP_NS_GU 2
#endif
#ifndef DG_EXP_KSP_DN
#define DG_EXP_KSP_DN 2
#endif
#ifndef DG_EXP_NS_DN
#define DG_EXP_NS_DN 2
#endif
// tile groups per workgroup (1 or 2) of the gate/up and down streams, and the k-tiles per wave and
// stage and register stages of the two-group form. Two groups halve the token bytes per weight
// byte; measured on the benchmark shapes, down 2-4 us faster with two, gate/up no faster.
#ifndef DG_EXP_GS_GU
#define DG_EXP_GS_GU 1
#endif
#ifndef DG_EXP_GS_DN
#define DG_EXP_GS_DN 2
#endif
#ifndef DG_EXP_KSP_GU2
#define DG_EXP_KSP_GU2 1
#endif
#ifndef DG_EXP_NS_GU2
#define DG_EXP_NS_GU2 2
#endif
#ifndef DG_EXP_KSP_DN2
#define DG_EXP_KSP_DN2 1
#endif
#ifndef DG_EXP_NS_DN2
#define DG_EXP_NS_DN2 2
#endif
constexpr int kExpWaves = 4;
#ifndef DG_EXP_NT
#define DG_EXP_NT 0
#endif
constexpr bool kExpNT = DG_EXP_NT;  // nontemporal weight loads
#ifndef DG_EXP_ROT
#define DG_EXP_ROT 0
#endif
constexpr bool kExpRot = DG_EXP_ROT;  // per-workgroup rotation of the stage order
#ifndef DG_EXP_MAX_NT
#define DG_EXP_MAX_NT 4
#endif
// 16-token tiles one pass of an expert workgroup holds: an expert with more tokens streams its
// weights once per pass, so the bound trades registers (accumulators) against weight re-reads.
// Four tiles fit two waves per SIMD when the accumulators live in ordinary VGPRs (the build
// compiles this file so); 48 tokens per pass measured 1 % slower on the benchmark routing.
constexpr int kExpMaxNT = DG_EXP_MAX_NT;

// Calls f(std::integral_constant<int, NT>) with the fewest 16-token tiles (at most kExpMaxNT)
// that cover `rem` tokens.
template <typename F>
__device__ inline void with_token_tiles(int rem, F&& f) {
  if constexpr (kExpMaxNT >= 4)
    if (rem > 48) return f(std::integral_constant<int, 4>());
  if constexpr (kExpMaxNT >= 3)
    if (rem > 32) return f(std::integral_constant<int, 3>());
  if (rem > 16) return f(std::integral_constant<int, 2>());
  f(std::integral_constant<int, 1>());
}

// Block b of an expert grid -> (expert, unit within the expert). Blocks are dispatched about in
// index order; with `rank` (offsets + E + 1: the experts, most tokens first) the experts are taken
// in that order, so an expert whose tokens take several passes over its weights starts early
// instead of finishing last (gate/up, measured 4 % faster with a skewed routing; down, whose
// units are a quarter as long, measured 3 % slower and keeps the index order). Workgroups of one
// expert read the same token rows, so with E a multiple of 8 they are kept on one XCD (the
// dispatcher sends block b to XCD b % 8).
__device__ inline void expert_of_block(int b, int per_e, int E, const int32_t* rank, int* e, int* q) {
  int r;
  if ((E & 7) == 0) {
    const int x = b & 7, j = b >> 3;
    r = (j / per_e) * 8 + x;
    *q = j % per_e;
  } else {
    r = b / per_e;
    *q = b % per_e;
  }
  *e = rank ? rank[r] : r;
}

// The 4 waves' partial sums of token tile t meet in LDS (red: 4 * G * 64 f32x4): every wave
// stores its own, then each output tile is summed by one wave, wave 0's partial first and then
// waves 1, 2, 3 in order.
template <int G, int NT>
__device__ inline void stash_partials(const f32x4_t (&acc)[G][NT], int t, f32x4_t* red, int wave, int lane) {
#pragma unroll
  for (int g = 0; g < G; ++g) red[(wave * G + g) * 64 + lane] = acc[g][t];
  __syncthreads();
}

template <int G>
__device__ inline f32x4_t sum_partials(const f32x4_t* red, int g, int lane) {
  f32x4_t v = red[g * 64 + lane];
#pragma unroll
  for (int w = 1; w < kExpWaves; ++w) v += red[(w * G + g) * 64 + lane];
  return v;
}

// One pass of a workgroup over GS consecutive tile groups of its expert's weights (G tiles per
// k-tile each, tiles.h; GS G tiles per k-step in all) against NT 16-token tiles. The k-tiles are
// split over the 4 waves in runs of KSP: stage s of wave w holds k-tiles
// s * 4 KSP + w KSP + u (u < KSP), so the four waves' loads of one stage
// cover 4 KSP consecutive k-tiles of the group, one contiguous run of memory
// (whole DRAM pages rather than scattered pieces of them; one run per group). Every token
// fragment feeds GS G products, so with GS = 2 a workgroup loads half the token bytes per weight
// byte that one group does (the expert's tokens are re-read by each of its workgroups). Weight and token
// fragments stream through NS register stages. Loads are never predicated
// (k-tiles past the end re-read the last one and are not multiplied; token
// rows past the expert's count repeat its last token and are not stored),
// so the compiler keeps exactly NS - 1 stages of loads outstanding. Each
// wave ends with the partial sums of its k-tiles.
template <typename T, int G, int NT, int KSP, int NS, int GS = 1>
struct SplitStream {
  using Fr = Frag<T>;
  using FT = typename Fr::type;
  static constexpr int GT = GS * G;  // weight tiles per k-step
  struct Stage {
    FT b[KSP][GT];
    FT a[KSP][NT];
  };
  f32x4_t acc[GT][NT];

  // bt: this lane's fragment in k-tile 0 of the first group; arow[t]: this lane's
  // token row of tile t at column 8 * (lane / 16); KT: k-tiles of 32.
  // rot: the stream starts at stage rot and wraps (workgroups running side by side then read
  // different offsets of their groups instead of marching through the same address bits together)
  __device__ inline void run(const T* bt, const T* const* arow, int KT, int wave, int rot) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[g][t] = f32x4_t{0, 0, 0, 0};
    constexpr int kPer = kExpWaves * KSP;
    const int nst = (KT + kPer - 1) / kPer;
    const int first = wave * KSP;
    const int64_t gstride = static_cast<int64_t>(KT) * G * kTileElems;  // one group's elements
    rot %= nst;
    auto rs = [&](int s) { const int r = s + rot; return r >= nst ? r - nst : r; };
    auto load = [&](Stage& S, int s) {
      const int base = rs(min(s, nst - 1)) * kPer + first;
#pragma unroll
      for (int u = 0; u < KSP; ++u) {
        const int kt = min(base + u, KT - 1);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const T* bp = bt + (g / G) * gstride + (static_cast<int64_t>(kt) * G + g % G) * kTileElems;
          S.b[u][g] = kExpNT ? Fr::load_nt(bp) : Fr::load(bp);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) S.a[u][t] = Fr::load(arow[t] + kt * 32);
      }
    };
    auto compute = [&](const Stage& S, int s) {
      const int base = rs(s) * kPer + first;
#pragma unroll
      for (int u = 0; u < KSP; ++u)
        if (base + u < KT) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int g = 0; g < GT; ++g) acc[g][t] = Fr::mma(S.a[u][t], S.b[u][g], acc[g][t]);
        }
    };
    Stage st[NS];
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) load(st[u], u);
    int s0 = 0;
    for (; s0 + NS <= nst; s0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        load(st[(u + NS - 1) % NS], s0 + u + NS - 1);
        compute(st[u], s0 + u);
      }
    }
    // tail: the remaining (< NS) stages are already loaded
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (s0 + u < nst) compute(st[u], s0 + u);
  }

  static constexpr int kTiles = GT;
  __device__ inline void stash(int t, f32x4_t* red, int wave, int lane) {
    stash_partials<GT, NT>(acc, t, red, wave, lane);
  }
};

#ifndef DG_EXP8_KP_GU
#define DG_EXP8_KP_GU 1
#endif
#ifndef DG_EXP8_NS_GU
#define DG_EXP8_NS_GU 2
#endif
#ifndef DG_EXP8_KP_DN
#define DG_EXP8_KP_DN 1
#endif
#ifndef DG_EXP8_NS_DN
#define DG_EXP8_NS_DN 2
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// 8 E4M3 codes (two dwords, code j in byte j) -> the bf16 B fragment of one k-step. Every E4M3
// value is exact in bf16 (3 fraction bits, exponents 2^-9 .. 2^8), so with a unit scale the
// conversion is exact; the per-row scale multiplies the fp32 accumulators instead.
__device__ inline bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  const bf16x4_t lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4_t hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// SplitStream over FP8 weights in the paired-tile order (tiles.h): the unit of the split is a
// pair of k-tiles, whose G blocks arrive as one 16-byte load per lane each (a contiguous
// kilobyte per wave, as in the bf16 stream); stage s of wave w holds pairs s * 4 KP + w KP + u.
// The token fragments stay bf16. Same unpredicated-load discipline as SplitStream.
template <int G, int NT, int KP, int NS>
struct SplitStream8 {
  using Fr = Frag<bf16_t>;
  struct Stage {
    u32x4v_t b[KP][G];
    bf16x8_t a[2 * KP][NT];
  };
  f32x4_t acc[G][NT];

  // bt: this lane's 16 bytes of pair 0 of the group; arow[t]: as in SplitStream; KT even.
  __device__ inline void run(const uint8_t* bt, const bf16_t* const* arow, int KT, int wave, int rot) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[g][t] = f32x4_t{0, 0, 0, 0};
    const int NP = KT / 2;
    constexpr int kPer = kExpWaves * KP;
    const int nst = (NP + kPer - 1) / kPer;
    const int first = wave * KP;
    rot %= nst;
    auto rs = [&](int s) { const int r = s + rot; return r >= nst ? r - nst : r; };
    auto load = [&](Stage& S, int s) {
      const int base = rs(min(s, nst - 1)) * kPer + first;
#pragma unroll
      for (int u = 0; u < KP; ++u) {
        const int p = min(base + u, NP - 1);
#pragma unroll
        for (int g = 0; g < G; ++g)
          S.b[u][g] = *reinterpret_cast<const u32x4v_t*>(bt + (static_cast<int64_t>(p) * G + g) * 1024);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < NT; ++t) S.a[2 * u + h][t] = Fr::load(arow[t] + (2 * p + h) * 32);
      }
    };
    auto compute = [&](const Stage& S, int s) {
      const int base = rs(s) * kPer + first;
#pragma unroll
      for (int u = 0; u < KP; ++u)
        if (base + u < NP) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const bf16x8_t bf = fp8x8_to_bf16(S.b[u][g][2 * h], S.b[u][g][2 * h + 1]);
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[g][t] = Fr::mma(S.a[2 * u + h][t], bf, acc[g][t]);
            }
        }
    };
    Stage st[NS];
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) load(st[u], u);
    int s0 = 0;
    for (; s0 + NS <= nst; s0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        load(st[(u + NS - 1) % NS], s0 + u + NS - 1);
        compute(st[u], s0 + u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (s0 + u < nst) compute(st[u], s0 + u);
  }

  static constexpr int kTiles = G;
  __device__ inline void stash(int t, f32x4_t* red, int wave, int lane) {
    stash_partials<G, NT>(acc, t, red, wave, lane);
  }
};

// act[slot][j] = GeLU(h W_gate[e]^T)_j * (h W_up[e]^T)_j (gated) or GeLU(h W_up[e]^T)_j for up to
// 16 NT slots of expert e starting at p0 and the 16 kGuBlocks GS features j0 .. of GS tile groups.
// FP8 (GS = 1): bt points at E4M3 codes and the products are multiplied by this lane's row scales
// scl[g] (gate blocks, then up blocks) before the activation.
template <typename T, bool GATED, int NT, bool FP8, int GS = 1>
__device__ inline void gateup_pass(const T* h, int64_t ldh, const void* bt, int F, int KT, int beg, int cnt, int p0,
                                   const int32_t* perm, T* act, int j0, int wave, int lane, f32x4_t* red,
                                   const float* scl) {
  constexpr int G = (GATED ? 2 : 1) * kGuBlocks;
  static_assert(!FP8 || GS == 1, "the FP8 stream covers one tile group");
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const T* arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int s = min(p0 + t * 16 + fr, cnt - 1);
    arow[t] = h + static_cast<int64_t>(perm[beg + s]) * ldh + fk;
  }
  std::conditional_t<FP8, SplitStream8<G, NT, DG_EXP8_KP_GU, DG_EXP8_NS_GU>,
                     std::conditional_t<GS == 1, SplitStream<T, G, NT, DG_EXP_KSP_GU, DG_EXP_NS_GU>,
                                        SplitStream<T, G, NT, DG_EXP_KSP_GU2, DG_EXP_NS_GU2, GS>>> sp;
  if constexpr (FP8) sp.run(static_cast<const uint8_t*>(bt), arow, KT, wave, kExpRot ? blockIdx.x : 0);
  else sp.run(static_cast<const T*>(bt), arow, KT, wave, kExpRot ? blockIdx.x : 0);
  constexpr int GT = decltype(sp)::kTiles;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sp.stash(t, red, wave, lane);
    // output tile pair pi (gate block, up block) is summed and stored by wave pi % 4
#pragma unroll
    for (int pi = 0; pi < GS * kGuBlocks; ++pi) {
      if (pi % kExpWaves != wave) continue;
      const int gi = pi / kGuBlocks, b = pi % kGuBlocks;
      const int ga = gi * G + b, gb = gi * G + kGuBlocks + b;
      const f32x4_t xg = sum_partials<GT>(red, ga, lane);
      const f32x4_t xu = GATED ? sum_partials<GT>(red, gb, lane) : xg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = p0 + t * 16 + (lane >> 4) * 4 + i;
        if (s < cnt) {
          const float a0 = FP8 ? xg[i] * scl[ga] : xg[i];
          const float v = GATED ? gelu_erf(a0) * (FP8 ? xu[i] * scl[gb] : xu[i]) : gelu_erf(a0);
          act[static_cast<int64_t>(beg + s) * F + j0 + pi * 16 + fr] = from_f32<T>(v);
        }
      }
    }
    __syncthreads();  // red is reused by the next tile or pass
  }
}

// Grid: E * (F / (16 kGuBlocks GS)) workgroups of 4 waves; block q of expert e owns feature groups
// GS q .. GS q + GS - 1.
template <typename T, bool GATED, int GS>
__global__ __launch_bounds__(256) void expert_gateup_kernel(
    const T* __restrict__ h, int64_t ldh, const T* __restrict__ w_gu, int E, int F, int D, int per_e,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, T* __restrict__ act) {
  constexpr int G = (GATED ? 2 : 1) * kGuBlocks;
  __shared__ f32x4_t red[kExpWaves * GS * G * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, q;
  expert_of_block(blockIdx.x, per_e, E, offsets + E + 1, &e, &q);
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int KT = D / 32;
  const T* bt = w_gu + static_cast<int64_t>(e) * (GATED ? 2 : 1) * F * D +
                static_cast<int64_t>(q) * GS * KT * G * kTileElems + lane * 8;
  const int j0 = q * GS * 16 * kGuBlocks;
  for (int p0 = 0; p0 < cnt; p0 += 16 * kExpMaxNT)
    with_token_tiles(cnt - p0, [&](auto nt) {
      gateup_pass<T, GATED, decltype(nt)::value, false, GS>(h, ldh, bt, F, KT, beg, cnt, p0, perm, act, j0, wave,
                                                            lane, red, nullptr);
    });
}

// The same over FP8 codes (paired tiles, tiles.h) with per-row scales sc[E][gw][F].
template <bool GATED>
__global__ __launch_bounds__(256) void expert_gateup_fp8_kernel(
    const bf16_t* __restrict__ h, int64_t ldh, const uint8_t* __restrict__ q_gu, const float* __restrict__ sc, int E,
    int F, int D, int per_e, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    bf16_t* __restrict__ act) {
  constexpr int gw = GATED ? 2 : 1;
  constexpr int G = gw * kGuBlocks;
  __shared__ f32x4_t red[kExpWaves * G * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, q;
  expert_of_block(blockIdx.x, per_e, E, offsets + E + 1, &e, &q);
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int KT = D / 32;
  const int j0 = q * 16 * kGuBlocks;
  float scl[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    scl[g] = sc[(static_cast<int64_t>(e) * gw + g / kGuBlocks) * F + j0 + (g % kGuBlocks) * 16 + (lane & 15)];
  const uint8_t* bt = q_gu + static_cast<int64_t>(e) * gw * F * D + static_cast<int64_t>(q) * KT * G * kTileElems +
                      lane * 16;
  for (int p0 = 0; p0 < cnt; p0 += 16 * kExpMaxNT)
    with_token_tiles(cnt - p0, [&](auto nt) {
      gateup_pass<bf16_t, GATED, decltype(nt)::value, true>(h, ldh, bt, F, KT, beg, cnt, p0, perm, act, j0, wave,
                                                            lane, red, scl);
    });
}

// out[slot][n] = gate[slot] * sum_f act[slot][f] W_down[e][n][f] for the 16 kDownGroup GS outputs n0 ..
// FP8 (GS = 1): bt points at E4M3 codes and output row block g is multiplied by this lane's row
// scale scl[g].
template <typename T, int NT, bool FP8, int GS = 1>
__device__ inline void down_pass(const T* act, const void* bt, int F, int D, int beg, int cnt, int p0,
                                 const float* slot_gate, float* out, int n0, int wave, int lane, f32x4_t* red,
                                 const float* scl) {
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const T* arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int s = min(p0 + t * 16 + fr, cnt - 1);
    arow[t] = act + static_cast<int64_t>(beg + s) * F + fk;
  }
  static_assert(!FP8 || GS == 1, "the FP8 stream covers one tile group");
  std::conditional_t<FP8, SplitStream8<kDownGroup, NT, DG_EXP8_KP_DN, DG_EXP8_NS_DN>,
                     std::conditional_t<GS == 1, SplitStream<T, kDownGroup, NT, DG_EXP_KSP_DN, DG_EXP_NS_DN>,
                                        SplitStream<T, kDownGroup, NT, DG_EXP_KSP_DN2, DG_EXP_NS_DN2, GS>>> sp;
  if constexpr (FP8) sp.run(static_cast<const uint8_t*>(bt), arow, F / 32, wave, kExpRot ? blockIdx.x : 0);
  else sp.run(static_cast<const T*>(bt), arow, F / 32, wave, kExpRot ? blockIdx.x : 0);
  constexpr int GT = decltype(sp)::kTiles;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sp.stash(t, red, wave, lane);
    float gs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) gs[i] = slot_gate[beg + min(p0 + t * 16 + (lane >> 4) * 4 + i, cnt - 1)];
    // output tile g is summed and stored by wave g % 4
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (g % kExpWaves != wave) continue;
      const f32x4_t x = sum_partials<GT>(red, g, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = p0 + t * 16 + (lane >> 4) * 4 + i;
        if (s < cnt) out[static_cast<int64_t>(beg + s) * D + n0 + g * 16 + fr] = gs[i] * (FP8 ? x[i] * scl[g] : x[i]);
      }
    }
    __syncthreads();  // red is reused by the next tile or pass
  }
}

// Grid: E * (D / (16 kDownGroup GS)) workgroups of 4 waves; block q of expert e owns output groups
// GS q .. GS q + GS - 1.
template <typename T, int GS>
__global__ __launch_bounds__(256) void expert_down_kernel(
    const T* __restrict__ act, const T* __restrict__ w_down, int E, int F, int D, int per_e,
    const int32_t* __restrict__ offsets, const float* __restrict__ slot_gate, float* __restrict__ out) {
  __shared__ f32x4_t red[kExpWaves * GS * kDownGroup * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, q;
  expert_of_block(blockIdx.x, per_e, E, nullptr, &e, &q);
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int KT = F / 32;
  const T* bt = w_down + static_cast<int64_t>(e) * D * F +
                static_cast<int64_t>(q) * GS * KT * kDownGroup * kTileElems + lane * 8;
  const int n0 = q * GS * kDownGroup * 16;
  for (int p0 = 0; p0 < cnt; p0 += 16 * kExpMaxNT)
    with_token_tiles(cnt - p0, [&](auto nt) {
      down_pass<T, decltype(nt)::value, false, GS>(act, bt, F, D, beg, cnt, p0, slot_gate, out, n0, wave, lane,
                                                   red, nullptr);
    });
}

// The same over FP8 codes (paired tiles, tiles.h) with per-row scales sc[E][D].
__global__ __launch_bounds__(256) void expert_down_fp8_kernel(
    const bf16_t* __restrict__ act, const uint8_t* __restrict__ q_down, const float* __restrict__ sc, int E, int F,
    int D, int per_e, const int32_t* __restrict__ offsets, const float* __restrict__ slot_gate,
    float* __restrict__ out) {
  __shared__ f32x4_t red[kExpWaves * kDownGroup * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, q;
  expert_of_block(blockIdx.x, per_e, E, nullptr, &e, &q);
  const int beg = offsets[e], cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;
  const int KT = F / 32;
  const int n0 = q * kDownGroup * 16;
  float scl[kDownGroup];
#pragma unroll
  for (int g = 0; g < kDownGroup; ++g) scl[g] = sc[static_cast<int64_t>(e) * D + n0 + g * 16 + (lane & 15)];
  const uint8_t* bt = q_down + static_cast<int64_t>(e) * D * F +
                      static_cast<int64_t>(q) * KT * kDownGroup * kTileElems + lane * 16;
  for (int p0 = 0; p0 < cnt; p0 += 16 * kExpMaxNT)
    with_token_tiles(cnt - p0, [&](auto nt) {
      down_pass<bf16_t, decltype(nt)::value, true>(act, bt, F, D, beg, cnt, p0, slot_gate, out, n0, wave, lane, red,
                                                   scl);
    });
}

// ------------------------------------------------------------ token-tiled experts (prefill chunks)
// With a prefill chunk of thousands of rows an expert holds hundreds of tokens, and the product is
// worth tiling like a dense GEMM rather than streaming the weights once per 48 tokens: a workgroup
// takes one entry of the tile list (128 of one expert's tokens) against one tile group of its
// weights (gate/up: 32 features of gate and up; down: 64 outputs) and runs K in stages of 64
// through an LDS ring filled by asynchronous copies: the 128 gathered token rows (128-byte
// rows, XOR-swizzled as in the dense GEMM) and the group's 2 G weight tiles (already in fragment
// order, so a lane reads its fragment at byte 16 l). Each of the 4 waves owns 32 tokens against
// all G weight tiles, so a wave holds both the gate and the up sums of its features.
#ifndef DG_TILE_STAGES
#define DG_TILE_STAGES 2
#endif
constexpr int kTileStages = DG_TILE_STAGES;  // LDS ring depth of the token-tiled experts
#ifndef DG_TILE_GROUPS
#define DG_TILE_GROUPS 1
#endif
// weight tile groups per workgroup: each adds 4 waves and the group's weight tiles to a stage, and
// divides the copies of the gathered token rows per flop by as much
constexpr int kTileGroups = DG_TILE_GROUPS;

// FP8: w holds E4M3 codes in the paired-tile order (tiles.h), whose 1 KiB block of a k-tile pair is
// exactly one 64-column stage of a tile; the codes are converted to bf16 fragments as they leave
// LDS and the row scales sc (gate/up [E][2][F], down [E][D]) multiply the sums in the epilogue.
template <bool DOWN, bool GATED, int NG, bool FP8>
__global__ __launch_bounds__(64 * kExpWaves * NG) void expert_tile_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const void* __restrict__ wv, int F, int D, int per_e,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
    const float* __restrict__ slot_gate, const float* __restrict__ sc, bf16_t* __restrict__ act,
    float* __restrict__ out) {
  using WT = std::conditional_t<FP8, uint8_t, bf16_t>;
  const WT* w = static_cast<const WT*>(wv);
  constexpr int NW = kExpWaves * NG;
  constexpr int gw = DOWN ? 1 : (GATED ? 2 : 1);
  constexpr int G = DOWN ? kDownGroup : gw * kGuBlocks;
  constexpr int KB = FP8 ? 1 : 2;                  // 1 KiB copies per weight tile and stage
  constexpr int ROWB = 128;                        // bytes per staged token row: 64 bf16
  constexpr int SA = kTileTokens * ROWB;           // token rows of a stage
  constexpr int SB = NG * KB * G * 1024;           // weight tiles of a stage (NG groups x 64 columns)
  constexpr int SS = SA + SB;
  constexpr int ALPW = kTileTokens / 8 / NW;       // token-row copies per wave per stage (8 rows each)
  constexpr int BLPW = NG * KB * G / NW;           // weight-tile copies per wave per stage
  constexpr int LPS = ALPW + BLPW;
  static_assert(ALPW >= 1 && BLPW >= 1 && (NG * KB * G) % NW == 0 && (kTileTokens / 8) % NW == 0,
                "copies of a stage must split evenly over the waves");
  __shared__ __align__(16) unsigned char smem[kTileStages * SS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = wave / kExpWaves, wq = wave % kExpWaves;  // this wave's group and 32-token quarter
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  const int ti = (j / per_e) * 8 + xcd, q = j % per_e;  // the tile's workgroups share an XCD (its L2)
  if (ti >= tiles[0]) return;
  const int entry = tiles[1 + ti];
  const int e = entry >> 16, t0 = (entry & 0xFFFF) * kTileTokens;
  const int beg = offsets[e], rows = min(kTileTokens, offsets[e + 1] - beg - t0);
  const int K = DOWN ? F : D;
  const int KT = K / 32, nk = K / 64;
  const WT* bg = w + static_cast<int64_t>(e) * (DOWN ? static_cast<int64_t>(D) * F : static_cast<int64_t>(gw) * F * D) +
                 static_cast<int64_t>(q) * NG * KT * G * kTileElems + lane * (FP8 ? 16 : 8);
  const bf16_t* asrc[ALPW];
#pragma unroll
  for (int i = 0; i < ALPW; ++i) {
    const int r = (wave * ALPW + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int slot = beg + t0 + min(r, rows - 1);  // rows past the tile's tokens repeat its last one
    const int64_t arow = DOWN ? slot : perm[slot];
    asrc[i] = A + arow * lda + c * 8;
  }
  auto issue = [&](int st, int slot) {
    unsigned char* base = smem + slot * SS;
#pragma unroll
    for (int i = 0; i < ALPW; ++i) dma16(asrc[i] + st * 64, base + (wave * ALPW + i) * 8 * ROWB);
#pragma unroll
    for (int i = 0; i < BLPW; ++i) {
      const int tb = wave * BLPW + i;  // group tb / (KB G), k-tile 2 st + (tb % (KB G)) / G, tile tb % G
      const int grp = tb / (KB * G), ks = (tb % (KB * G)) / G;
      if constexpr (FP8)  // the pair block of the stage: 1 KiB per tile
        dma16(bg + static_cast<int64_t>(grp) * KT * G * kTileElems + (static_cast<int64_t>(st) * G + tb % G) * 1024,
              base + SA + tb * 1024);
      else
        dma16(bg + (static_cast<int64_t>(grp) * KT * G + static_cast<int64_t>(2 * st + ks) * G + tb % G) * kTileElems,
              base + SA + tb * 1024);
    }
  };
  f32x4_t acc[2][G];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[t][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int st = 0; st < kTileStages - 1; ++st)
    if (st < nk) issue(st, st);
  for (int st = 0; st < nk; ++st) {
    wait_stages<LPS, kTileStages>(min(kTileStages - 2, nk - 1 - st));
    // stage st is in LDS for every wave and every wave has consumed stage st - 1 (a bare barrier:
    // the fence of __syncthreads() would drain the copies still in flight)
    __builtin_amdgcn_s_barrier();
    if (st + kTileStages - 1 < nk) issue(st + kTileStages - 1, (st + kTileStages - 1) % kTileStages);
    const unsigned char* sa = smem + (st % kTileStages) * SS;
    const unsigned char* sb = sa + SA + gi * KB * G * 1024;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[2], bfr[G];
      const int c = ks * 4 + g4;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = wq * 32 + t * 16 + fr;
        af[t] = *reinterpret_cast<const bf16x8_t*>(sa + r * ROWB + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (FP8) {
          const u32x4v_t v = *reinterpret_cast<const u32x4v_t*>(sb + g * 1024 + lane * 16);
          bfr[g] = fp8x8_to_bf16(v[2 * ks], v[2 * ks + 1]);
        } else {
          bfr[g] = *reinterpret_cast<const bf16x8_t*>(sb + (ks * G + g) * 1024 + lane * 16);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[t][g] = Frag<bf16_t>::mma(af[t], bfr[g], acc[t][g]);
    }
  }
  // epilogue: lane holds tokens wq * 32 + 16 t + 4 (lane / 16) + i of the tile, group row 16 g + lane % 16
  const int qg = q * NG + gi;  // this wave's tile group within the expert
  float scl[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (!FP8) scl[g] = 1.f;
    else if constexpr (DOWN) scl[g] = sc[static_cast<int64_t>(e) * D + qg * 16 * kDownGroup + g * 16 + fr];
    else scl[g] = sc[(static_cast<int64_t>(e) * gw + g / kGuBlocks) * F + qg * 16 * kGuBlocks + (g % kGuBlocks) * 16 + fr];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wq * 32 + t * 16 + g4 * 4 + i;
      if (r < rows) {
        const int64_t slot = beg + t0 + r;
        if constexpr (DOWN) {
          const float gs = slot_gate[slot];
          float* o = out + slot * D + qg * 16 * kDownGroup + fr;
#pragma unroll
          for (int g = 0; g < G; ++g) o[g * 16] = gs * (FP8 ? acc[t][g][i] * scl[g] : acc[t][g][i]);
        } else {
          bf16_t* o = act + slot * F + qg * 16 * kGuBlocks + fr;
#pragma unroll
          for (int bb = 0; bb < kGuBlocks; ++bb) {
            const float a0 = FP8 ? acc[t][bb][i] * scl[bb] : acc[t][bb][i];
            const float a1 = FP8 ? acc[t][kGuBlocks + bb][i] * scl[kGuBlocks + bb] : acc[t][kGuBlocks + bb][i];
            o[bb * 16] = f32_to_bf16(GATED ? gelu_erf(a0) * a1 : gelu_erf(a0));
          }
        }
      }
    }
}

template <bool DOWN, bool GATED, bool FP8>
static void launch_expert_tiles(int t8, int per_e, hipStream_t s, const bf16_t* A, int64_t lda, const void* w,
                                int F, int D, const int32_t* offsets, const int32_t* perm, const int32_t* tiles,
                                const float* slot_gate, const float* sc, bf16_t* act, float* out) {
  if (per_e % kTileGroups == 0)
    expert_tile_kernel<DOWN, GATED, kTileGroups, FP8><<<t8 * (per_e / kTileGroups), 64 * kExpWaves * kTileGroups, 0,
                                                        s>>>(A, lda, w, F, D, per_e / kTileGroups, offsets, perm,
                                                             tiles, slot_gate, sc, act, out);
  else
    expert_tile_kernel<DOWN, GATED, 1, FP8><<<t8 * per_e, 64 * kExpWaves, 0, s>>>(A, lda, w, F, D, per_e, offsets,
                                                                                perm, tiles, slot_gate, sc, act, out);
}

// ------------------------------------------------------------------- host
// tiles (may be null; needed for M > 256): the token-tile list of permute_kernel, 2 + M k / 128 + E ints
int moe_route(const float* part, int splits, int M, int E, int k, int renorm, float* rlog, int32_t* sel,
              float* gate, int32_t* offsets, int32_t* perm, int32_t* slot_of, float* slot_gate, int32_t* tiles,
              hipStream_t s) {
  if (M < 1 || M > kMaxTokensLarge || E > 256 || k > 16 || k > E || splits < 1 || splits > kRouteSplits)
    return fail(DG_ERR_UNSUPPORTED, "routing limits: 1<=M<=4096, E<=256, k<=min(16,E), at most 32 partials");
  if (M > kMaxTokens && E > 16384 / (kMaxTokensLarge / 32))
    return fail(DG_ERR_UNSUPPORTED, "routing more than 256 rows at once needs n_experts <= 128");
  {
    ProfScope ps("moe_topk", s);
    const unsigned g = (M + kRouteWaves - 1) / kRouteWaves, t = 64 * kRouteWaves;
    if (splits <= 8) route_topk_kernel<8><<<g, t, 0, s>>>(part, M, E, k, renorm, splits, rlog, sel, gate);
    else if (splits <= 16) route_topk_kernel<16><<<g, t, 0, s>>>(part, M, E, k, renorm, splits, rlog, sel, gate);
    else route_topk_kernel<kRouteSplits><<<g, t, 0, s>>>(part, M, E, k, renorm, splits, rlog, sel, gate);
  }
  DG_LAUNCH_CHECK("route_topk_kernel");
  {
    ProfScope ps("moe_permute", s);
    if (M <= kMaxTokens)
      permute_kernel<kMaxTokens / 32><<<1, 1024, 0, s>>>(sel, gate, M, E, k, offsets, perm, slot_of, slot_gate, tiles);
    else
      permute_kernel<kMaxTokensLarge / 32><<<1, 1024, 0, s>>>(sel, gate, M, E, k, offsets, perm, slot_of, slot_gate,
                                                              tiles);
  }
  DG_LAUNCH_CHECK("permute_kernel");
  return DG_OK;
}

// x[row][c] += y[row][c] + sum_j slot_out[slot_of[row * k + j]][c], j = 0 .. k-1 in order (the
// shared expert's output, then the token's gated routed outputs); four columns per thread
__global__ __launch_bounds__(256) void combine_kernel(float* __restrict__ x, const float* __restrict__ y,
                                                      const float* __restrict__ slot_out,
                                                      const int32_t* __restrict__ slot_of, int M, int D4, int k) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * D4) return;
  const int row = static_cast<int>(i / D4), c4 = static_cast<int>(i - static_cast<int64_t>(row) * D4);
  const float4* y4 = reinterpret_cast<const float4*>(y);
  const float4* so = reinterpret_cast<const float4*>(slot_out);
  float4 acc = y4[i];
  for (int j = 0; j < k; ++j) {
    const float4 v = so[static_cast<int64_t>(slot_of[row * k + j]) * D4 + c4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  float4* x4 = reinterpret_cast<float4*>(x);
  float4 xv = x4[i];
  xv.x += acc.x; xv.y += acc.y; xv.z += acc.z; xv.w += acc.w;
  x4[i] = xv;
}

int moe_combine(float* x, const float* y, const float* slot_out, const int32_t* slot_of, int M, int D, int k,
                hipStream_t s) {
  if (D % 4 != 0) return fail(DG_ERR_UNSUPPORTED, "combine: d_model must be a multiple of 4");
  const int64_t n = static_cast<int64_t>(M) * (D / 4);
  if (n == 0) return DG_OK;
  ProfScope ps("moe_combine", s);
  combine_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(x, y, slot_out, slot_of, M, D / 4, k);
  DG_LAUNCH_CHECK("combine_kernel");
  return DG_OK;
}

// q8 (optional): FP8 codes and scales of the same layer's routed experts; when given, the expert
// kernels stream those instead of w_gu / w_down (bf16 models only).
// tiles (optional, bf16 only): the token-tile list of moe_route for M rows; the experts then run as
// token-tiled GEMMs (M k / 128 + E tiles at most) instead of weight streams.
int moe_experts(const void* h, int64_t ldh, const void* w_gu, const void* w_down, int E, int F, int D, int gated,
                const int32_t* offsets, const int32_t* perm, const float* slot_gate, void* act, float* out,
                int dtype, const ExpertsFp8* q8, const int32_t* tiles, int M, int k, hipStream_t s) {
  if (F % (16 * kGuBlocks) != 0 || D % (16 * kDownGroup) != 0)
    return fail(DG_ERR_UNSUPPORTED, "expert width and d_model must be multiples of 32 and 64");
  const int per_gu = F / (16 * kGuBlocks);
  const int per_dn = D / (16 * kDownGroup);
  const dim3 g1(E * per_gu), g2(E * per_dn);
  // token tiles: bf16 weights, or FP8 codes of a gated model (an ungated one's G = 2 weight tiles per
  // stage do not split over 4 waves in whole kilobytes)
  if (tiles && dtype == DG_BF16 && (!q8 || gated)) {
    if (F % 64 != 0 || D % 64 != 0) return fail(DG_ERR_UNSUPPORTED, "token-tiled experts need widths that are multiples of 64");
    const int t8 = (static_cast<int>((static_cast<int64_t>(M) * k + kTileTokens - 1) / kTileTokens) + E + 7) / 8 * 8;
    const bf16_t* hh = static_cast<const bf16_t*>(h);
    bf16_t* a = static_cast<bf16_t*>(act);
    {
      ProfScope ps(q8 ? "expert_tile_gateup_fp8" : "expert_tile_gateup", s);
      if (q8)
        launch_expert_tiles<false, true, true>(t8, per_gu, s, hh, ldh, q8->gu, F, D, offsets, perm, tiles, slot_gate,
                                               q8->s_gu, a, out);
      else if (gated)
        launch_expert_tiles<false, true, false>(t8, per_gu, s, hh, ldh, w_gu, F, D, offsets, perm, tiles, slot_gate,
                                                nullptr, a, out);
      else
        launch_expert_tiles<false, false, false>(t8, per_gu, s, hh, ldh, w_gu, F, D, offsets, perm, tiles, slot_gate,
                                                 nullptr, a, out);
    }
    DG_LAUNCH_CHECK("expert_tile_kernel (gate/up)");
    {
      ProfScope ps(q8 ? "expert_tile_down_fp8" : "expert_tile_down", s);
      if (q8)
        launch_expert_tiles<true, false, true>(t8, per_dn, s, a, F, q8->dn, F, D, offsets, perm, tiles, slot_gate,
                                               q8->s_dn, a, out);
      else
        launch_expert_tiles<true, false, false>(t8, per_dn, s, a, F, w_down, F, D, offsets, perm, tiles, slot_gate,
                                                nullptr, a, out);
    }
    DG_LAUNCH_CHECK("expert_tile_kernel (down)");
    return DG_OK;
  }
  if (q8) {
    if (dtype != DG_BF16 || F % 64 != 0 || D % 64 != 0)
      return fail(DG_ERR_UNSUPPORTED, "FP8 experts need a bf16 model and widths that are multiples of 64");
    const bf16_t* hh = static_cast<const bf16_t*>(h);
    bf16_t* a = static_cast<bf16_t*>(act);
    {
      ProfScope ps("expert_gateup_fp8", s);
      if (gated) expert_gateup_fp8_kernel<true><<<g1, dim3(256), 0, s>>>(hh, ldh, q8->gu, q8->s_gu, E, F, D,
                              per_gu, offsets, perm, a);
      else expert_gateup_fp8_kernel<false><<<g1, dim3(256), 0, s>>>(hh, ldh, q8->gu, q8->s_gu, E, F, D,
                        per_gu, offsets, perm, a);
    }
    DG_LAUNCH_CHECK("expert_gateup_fp8_kernel");
    {
      ProfScope ps("expert_down_fp8", s);
      expert_down_fp8_kernel<<<g2, 256, 0, s>>>(a, q8->dn, q8->s_dn, E, F, D, per_dn, offsets, slot_gate, out);
    }
    DG_LAUNCH_CHECK("expert_down_fp8_kernel");
    return DG_OK;
  }
  {
    ProfScope ps("expert_gateup", s);
    // two groups per workgroup where the features split evenly (bf16 only: fp32 fragments take
    // twice the registers)
    constexpr bool kTwoGu = DG_EXP_GS_GU == 2;
    const bool two = kTwoGu && dtype == DG_BF16 && F % (32 * kGuBlocks) == 0;
    const dim3 g(two ? g1.x / 2 : g1.x);
    const int per = two ? per_gu / 2 : per_gu;
    if (dtype == DG_BF16) {
      const bf16_t* hh = static_cast<const bf16_t*>(h);
      const bf16_t* w = static_cast<const bf16_t*>(w_gu);
      bf16_t* a = static_cast<bf16_t*>(act);
      if constexpr (kTwoGu) {
        if (two) {
          if (gated) expert_gateup_kernel<bf16_t, true, 2><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
          else expert_gateup_kernel<bf16_t, false, 2><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
        }
      }
      if (!two) {
        if (gated) expert_gateup_kernel<bf16_t, true, 1><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
        else expert_gateup_kernel<bf16_t, false, 1><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
      }
    } else {
      const float* hh = static_cast<const float*>(h);
      const float* w = static_cast<const float*>(w_gu);
      float* a = static_cast<float*>(act);
      if (gated) expert_gateup_kernel<float, true, 1><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
      else expert_gateup_kernel<float, false, 1><<<g, 256, 0, s>>>(hh, ldh, w, E, F, D, per, offsets, perm, a);
    }
  }
  DG_LAUNCH_CHECK("expert_gateup_kernel");
  {
    ProfScope ps("expert_down", s);
    constexpr bool kTwoDn = DG_EXP_GS_DN == 2;
    const bool two = kTwoDn && dtype == DG_BF16 && D % (32 * kDownGroup) == 0;
    const dim3 g(two ? g2.x / 2 : g2.x);
    const int per = two ? per_dn / 2 : per_dn;
    if (dtype == DG_BF16) {
      const bf16_t* a = static_cast<const bf16_t*>(act);
      const bf16_t* w = static_cast<const bf16_t*>(w_down);
      if constexpr (kTwoDn) {
        if (two) expert_down_kernel<bf16_t, 2><<<g, 256, 0, s>>>(a, w, E, F, D, per, offsets, slot_gate, out);
      }
      if (!two) expert_down_kernel<bf16_t, 1><<<g, 256, 0, s>>>(a, w, E, F, D, per, offsets, slot_gate, out);
    } else {
      expert_down_kernel<float, 1><<<g, 256, 0, s>>>(static_cast<const float*>(act),
          static_cast<const float*>(w_down), E, F, D, per, offsets, slot_gate, out);
    }
  }
  DG_LAUNCH_CHECK("expert_down_kernel");
  return DG_OK;
}

}  // namespace dg
