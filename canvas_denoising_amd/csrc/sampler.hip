// Entropy-bounded sampler over the canvas logits, one read of the logits.
//
// [P3] "Inference mechanism": the logits scheduler sharpens with a
// temperature; the entropy-bounded sampler accepts tokens by an entropy-based
// confidence and re-noises the others with random tokens. [P4] "Standard
// sampling settings" (table) and "Two-Fold Adaptive Stopping" give the
// constants and the stop rule.
//
// Split-row design: a [rows x vocab] logits matrix has far too few rows for
// 256 CUs, so every row is cut into `splits` chunks. A workgroup streams one
// chunk once with 16-byte coalesced loads (the next batch is in flight while
// the current one is reduced) and reduces it to a record (m = max logit,
// Z = sum 2^u, A = sum u 2^u with u = (l - m) log2(e) / T, argmax). Records
// merge exactly:
//   m = max(m1, m2), d_i = (m_i - m) log2(e)/T,
//   Z = Z1 2^d1 + Z2 2^d2,  A = 2^d1 (A1 + d1 Z1) + 2^d2 (A2 + d2 Z2),
// and the row entropy is H = ln Z - ln2 * A / Z, so no second read is needed.
// A batch's maximum is a tree of maxima; each thread notes the batch in which
// its running maximum was last raised, and once the chunk maximum is known
// the threads holding it find its first position in that batch (the last two
// batches are still in registers), so the chunk's argmax is the lowest of
// those positions.
//
// A second, single-workgroup kernel merges each row's records in a fixed
// order (a quad of threads per row), applies the accept / Philox re-noise
// rule, and reduces the canvas mean entropy and the stability test in a
// fixed order into the stop state. (Folding this into
// the first kernel with a last-workgroup atomic costs a cache write-back and
// invalidate per workgroup at agent scope, far more than a second launch.)
// Results are bitwise reproducible.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "dg_common.h"
#include "entrec.h"
#include "philox.h"
#include "prof.h"

namespace dg {

// Categorical sampling: the best Gumbel-perturbed score of a chunk and its (lowest) index.
struct GRec {
  float s;
  int idx;
};

__device__ inline void gmax(float& bs, int& bi, float os, int oi) {
  if (os > bs || (os == bs && oi < bi)) { bs = os; bi = oi; }
}

// -ln(-ln u) for the 24-bit uniform u = (r >> 8 + 1/2) / 2^24 of Philox word r, with the hardware
// base-2 logarithm (u and -ln u are normal floats here: u >= 2^-25, -ln u >= 2^-25)
__device__ inline float gumbel_of(uint32_t r) {
  constexpr float kLn2f = 0.693147180559945309f;
  const float u = (static_cast<float>(r >> 8) + 0.5f) * 5.9604644775390625e-8f;
  const float e = -__builtin_amdgcn_logf(u) * kLn2f;  // -ln u > 0
  return -__builtin_amdgcn_logf(e) * kLn2f;
}

constexpr int kSampThreads = 256;
constexpr int kVec = 8;      // elements per 16-byte (bf16) / 32-byte (fp32) group
constexpr int kUnroll = 4;   // groups per thread per batch
constexpr int kBatch = kSampThreads * kVec * kUnroll;  // elements per workgroup batch
constexpr int kMaxSplits = 64;

// The two bf16 halves of a 32-bit word as floats, by the bf16 -> f32 conversion (exact, the same
// bits as a shift): converted values are known to be canonical floats, so the compiler takes their
// maxima without a quieting step per value.
__device__ inline float widen_lo(uint32_t w) { return static_cast<float>(__builtin_bit_cast(__bf16, static_cast<uint16_t>(w))); }
__device__ inline float widen_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(__bf16, static_cast<uint16_t>(w >> 16)));
}

// raw storage of one thread's batch: kUnroll groups of 8 elements
template <typename T> struct Raw;
// The logits are read once: nontemporal loads keep them from displacing reused lines in the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <> struct Raw<bf16_t> {
  uint4 q[kUnroll];
  __device__ inline void load(const bf16_t* p) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = load_nt(p + u * kSampThreads * kVec);
  }
  __device__ inline void unpack(float* v) const {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      v[u * 8 + 0] = widen_lo(q[u].x); v[u * 8 + 1] = widen_hi(q[u].x);
      v[u * 8 + 2] = widen_lo(q[u].y); v[u * 8 + 3] = widen_hi(q[u].y);
      v[u * 8 + 4] = widen_lo(q[u].z); v[u * 8 + 5] = widen_hi(q[u].z);
      v[u * 8 + 6] = widen_lo(q[u].w); v[u * 8 + 7] = widen_hi(q[u].w);
    }
  }
};
template <> struct Raw<float> {
  float4 q[2 * kUnroll];
  __device__ inline void load(const float* p) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      q[2 * u] = *reinterpret_cast<const float4*>(p + u * kSampThreads * kVec);
      q[2 * u + 1] = *reinterpret_cast<const float4*>(p + u * kSampThreads * kVec + 4);
    }
  }
  __device__ inline void unpack(float* v) const {
#pragma unroll
    for (int u = 0; u < 2 * kUnroll; ++u) {
      v[u * 4 + 0] = q[u].x; v[u * 4 + 1] = q[u].y; v[u * 4 + 2] = q[u].z; v[u * 4 + 3] = q[u].w;
    }
  }
};

template <typename T> __device__ inline float load1(const T* p);
template <> __device__ inline float load1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <> __device__ inline float load1<float>(const float* p) { return *p; }

// largest of N values (N a power of two) by a tree of maxima: exact, so it equals the first
// maximum of any order
template <int N>
__device__ inline float max_of(const float* v) {
  static_assert((N & (N - 1)) == 0, "power of two");
  float t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = v[j];
#pragma unroll
  for (int s = N / 2; s >= 1; s /= 2)
#pragma unroll
    for (int j = 0; j < s; ++j) t[j] = fmaxf(t[j], t[j + s]);
  return t[0];
}

// the first j with v[j] == m, for an m that is one of the N values
template <int N>
__device__ inline int first_of(const float* v, float m) {
  int bj = N - 1;
#pragma unroll
  for (int j = N - 2; j >= 0; --j)
    if (v[j] == m) bj = j;
  return bj;
}

// fold N values into the running (m, z, a); returns true when the running max grew
template <int N>
__device__ inline bool fold(const float* v, float c, Rec& r) {
  const float bm = max_of<N>(v);
  bool grew = false;
  if (bm > r.m) {
    if (r.z != 0.f) {
      const float d = (r.m - bm) * c;
      const float s = __builtin_amdgcn_exp2f(d);
      r.a = s * (r.a + d * r.z);
      r.z *= s;
    }
    r.m = bm;
    grew = true;
  }
  const float off = -r.m * c;
  float z = 0.f, a = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float u = fmaf(v[j], c, off);
    const float e = __builtin_amdgcn_exp2f(u);
    z += e;
    a = fmaf(u, e, a);
  }
  r.z += z;
  r.a += a;
  return grew;
}

struct SampleArgs {
  const void* logits;
  int64_t vocab;
  int64_t chunk;
  int rows, splits;
  float c;  // log2(e) / T
  float bound, stop_thr;
  int stable_needed;
  int mode;  // DG_SCHED_* flags
  float inv_t;  // 1 / T (categorical sampling)
  uint64_t seed;
  int step, block;
  int32_t* canvas;
  int32_t* pred;
  uint8_t* accept;
  float* entropy;
  float* row_stats;
  dg_stop_state* stop;
  Rec* recs;    // scratch [rows][splits]
  GRec* grecs;  // scratch [rows][splits] (categorical sampling)
};

// Gumbel scores of the 8 tokens e0 .. e0+7 (e0 % 8 == 0) of `row`, folded into (bs, bi)
__device__ inline void gumbel_fold8(const SampleArgs& g, int row, int64_t e0, const float* v, float& bs, int& bi) {
  const uint32_t k0 = static_cast<uint32_t>(g.seed), k1 = static_cast<uint32_t>(g.seed >> 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t q = static_cast<uint32_t>((e0 >> 2) + h);
    const PhiloxOut o = philox4x32_10(static_cast<uint32_t>(row), static_cast<uint32_t>(g.step),
                                      static_cast<uint32_t>(g.block), kPurposeGumbel + 4u * q, k0, k1);
    const uint32_t w[4] = {o.w0, o.w1, o.w2, o.w3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = fmaf(v[h * 4 + j], g.inv_t, gumbel_of(w[j]));
      if (sc > bs) { bs = sc; bi = static_cast<int>(e0 + h * 4 + j); }  // ascending positions: first max kept
    }
  }
}

// grid (splits, rows)
template <typename T, bool kVecPath, bool CAT>
__global__ __launch_bounds__(kSampThreads) void sample_kernel(SampleArgs g) {
  if (g.stop->stopped) return;
  const int sp = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float c = g.c;
  const int64_t begin = sp * g.chunk;
  const int64_t end = min(begin + g.chunk, g.vocab);
  const T* p = static_cast<const T*>(g.logits) + static_cast<int64_t>(row) * g.vocab;
  Rec r{-INFINITY, 0.f, 0.f, 0x7FFFFFFF};
  __shared__ Rec sh[kSampThreads / 64];
  __shared__ int sh_idx[kSampThreads / 64];

  if (kVecPath) {
    // whole batches, software-pipelined: batch b+1 is loaded while batch b is folded
    const int64_t nb = (end - begin) / kBatch;
    const T* tp = p + begin + static_cast<int64_t>(tid) * kVec;
    float gs = -INFINITY;  // categorical: best Gumbel score of this thread and its index
    int gi = 0x7FFFFFFF;
    auto gumbel_batch = [&](const float* v, int64_t b) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        gumbel_fold8(g, row, begin + b * kBatch + static_cast<int64_t>(tid) * kVec + u * kSampThreads * kVec,
                     v + u * kVec, gs, gi);
    };
    // element j of a thread's batch b is token begin + b kBatch + (j / 8) 2048 + 8 tid + j % 8
    auto token = [&](int64_t b, int j) {
      return static_cast<int>(begin + b * kBatch + (j / kVec) * kSampThreads * kVec + static_cast<int64_t>(tid) * kVec +
                              (j % kVec));
    };
    // qa holds the even batches, qb the odd ones; bbest is the batch in which this thread's running
    // maximum was last raised (-1 once the tail raised it: r.idx is then set)
    Raw<T> qa, qb;
    int64_t bbest = -1;
    if (nb > 0) qa.load(tp);
    for (int64_t b = 0; b < nb; b += 2) {
      if (b + 1 < nb) qb.load(tp + (b + 1) * kBatch);
      {
        float v[kUnroll * kVec];
        qa.unpack(v);
        if (fold<kUnroll * kVec>(v, c, r)) bbest = b;
        if constexpr (CAT) gumbel_batch(v, b);
      }
      if (b + 1 < nb) {
        if (b + 2 < nb) qa.load(tp + (b + 2) * kBatch);
        float v[kUnroll * kVec];
        qb.unpack(v);
        if (fold<kUnroll * kVec>(v, c, r)) bbest = b + 1;
        if constexpr (CAT) gumbel_batch(v, b + 1);
      }
    }
    // tail: whole groups of 8 (vocab % 8 == 0 on this path), index tracked directly
    const int64_t tail0 = begin + nb * kBatch;
    for (int64_t e0 = tail0 + static_cast<int64_t>(tid) * kVec; e0 < end; e0 += static_cast<int64_t>(kSampThreads) * kVec) {
      float v[kVec];
      if constexpr (sizeof(T) == 2) {
        const uint4 q = *reinterpret_cast<const uint4*>(p + e0);
        v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
        v[4] = bf16lo(q.z); v[5] = bf16hi(q.z); v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) v[j] = load1<T>(p + e0 + j);
      }
      float bm = v[0];
      int bj = 0;
#pragma unroll
      for (int j = 1; j < kVec; ++j)
        if (v[j] > bm) { bm = v[j]; bj = j; }
      if (fold<kVec>(v, c, r)) {
        r.idx = static_cast<int>(e0 + bj);
        bbest = -1;
      }
      if constexpr (CAT) gumbel_fold8(g, row, e0, v, gs, gi);
    }
    if constexpr (CAT) {  // the chunk's best Gumbel score: wave (DPP / row swaps), then the 4 waves
      gmax(gs, gi, dpp_f32<kDppXor1>(gs), static_cast<int>(dpp_u32<kDppXor1>(static_cast<uint32_t>(gi))));
      gmax(gs, gi, dpp_f32<kDppXor2>(gs), static_cast<int>(dpp_u32<kDppXor2>(static_cast<uint32_t>(gi))));
      gmax(gs, gi, dpp_f32<kDppHalfMirror>(gs), static_cast<int>(dpp_u32<kDppHalfMirror>(static_cast<uint32_t>(gi))));
      gmax(gs, gi, dpp_f32<kDppMirror>(gs), static_cast<int>(dpp_u32<kDppMirror>(static_cast<uint32_t>(gi))));
      gmax(gs, gi, xrow16_f32(gs), static_cast<int>(xrow16_u32(static_cast<uint32_t>(gi))));
      gmax(gs, gi, xrow32_f32(gs), static_cast<int>(xrow32_u32(static_cast<uint32_t>(gi))));
      __shared__ GRec shg[kSampThreads / 64];
      if (lane == 0) shg[wave] = GRec{gs, gi};
      __syncthreads();
      if (tid == 0) {
        GRec best = shg[0];
#pragma unroll
        for (int i = 1; i < kSampThreads / 64; ++i) gmax(best.s, best.idx, shg[i].s, shg[i].idx);
        g.grecs[static_cast<int64_t>(row) * g.splits + sp] = best;
      }
    }
    // wave / workgroup merge of (m, z, a) in a fixed order
    Rec w = r;
    rec_wave_merge(w, c);
    if (lane == 0) sh[wave] = w;
    __syncthreads();
    Rec tot = sh[0];
#pragma unroll
    for (int i = 1; i < kSampThreads / 64; ++i) rec_merge(tot, sh[i], c);
    // argmax: lowest index holding the chunk maximum. A thread holding it finds the first position
    // of its maximum in the batch where that was raised (values in increasing index order, and an
    // equal value in a later batch did not raise it); the last two batches are still in registers.
    const bool holds = r.z != 0.f && r.m == tot.m;
    if (holds && bbest >= 0) {
      Raw<T> q;
      if (bbest >= nb - 2) q = (bbest % 2 == 0) ? qa : qb;
      else q.load(tp + bbest * kBatch);
      float v[kUnroll * kVec];
      q.unpack(v);
      r.idx = token(bbest, first_of<kUnroll * kVec>(v, r.m));
    }
    const int my_idx = holds ? r.idx : 0x7FFFFFFF;
    const int w_idx = wave_min_i32(my_idx);
    if (lane == 0) sh_idx[wave] = w_idx;
    __syncthreads();
    if (tid == 0) {
      int bi = sh_idx[0];
#pragma unroll
      for (int i = 1; i < kSampThreads / 64; ++i) bi = min(bi, sh_idx[i]);
      tot.idx = bi;
      g.recs[static_cast<int64_t>(row) * g.splits + sp] = tot;
    }
  } else {
    // scalar path (vocab not a multiple of 8): index tracked per element
    for (int64_t e = begin + tid; e < end; e += kSampThreads) {
      float v[1] = {load1<T>(p + e)};
      if (fold<1>(v, c, r)) r.idx = static_cast<int>(e);
    }
    rec_wave_merge(r, c);
    if (lane == 0) sh[wave] = r;
    __syncthreads();
    if (tid == 0) {
      Rec tot = sh[0];
      for (int i = 1; i < kSampThreads / 64; ++i) rec_merge(tot, sh[i], c);
      g.recs[static_cast<int64_t>(row) * g.splits + sp] = tot;
    }
  }

}

constexpr int kFinThreads = 1024;
constexpr int kGroupMaxRows = 4096;  // rows the group acceptance ranks in LDS

__device__ inline int32_t renoise_token(const SampleArgs& g, int row) {
  return draw_token(g.seed, static_cast<uint32_t>(row), static_cast<uint32_t>(g.step), static_cast<uint32_t>(g.block),
                    kPurposeRenoise, static_cast<uint32_t>(g.vocab));
}
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinParts = 4;                     // threads per row (one DPP quad)
constexpr int kFinRecs = kMaxSplits / kFinParts;  // records per thread at most

// One workgroup; a quad of threads per row, 256 rows per pass. Thread part p of a row loads the
// records p, p + 4, ... (all loads issued before any merge: one memory round trip) and merges them
// in increasing order; the quad then merges its four partial records (lane ^ 1, then lane ^ 2) and
// part 0 finalises the row (accept, Philox re-noise, outputs). The canvas mean entropy, the
// stability test and the stop rule are reduced in a fixed order at the end.
__global__ __launch_bounds__(kFinThreads) void sample_finalize_kernel(SampleArgs g) {
  if (g.stop->stopped) return;
  __shared__ float shs[kFinWaves];
  __shared__ int shq[kFinWaves];
  __shared__ float gH[kGroupMaxRows];    // group acceptance: entropy per row, then in rank order
  __shared__ int32_t gIdx[kGroupMaxRows];
  __shared__ int gK;
  const bool group = (g.mode & DG_SCHED_ACCEPT_GROUP) != 0;
  const bool cat = (g.mode & DG_SCHED_SAMPLE) != 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = tid % kFinParts;
  const float c = g.c;
  float hs = 0.f;
  int same = 1;
  for (int base = 0; base < g.rows; base += kFinThreads / kFinParts) {
    const int row = base + tid / kFinParts;
    const bool valid = row < g.rows;
    Rec buf[kFinRecs];
#pragma unroll
    for (int i = 0; i < kFinRecs; ++i) {
      const int sp = part + kFinParts * i;
      buf[i] = Rec{-INFINITY, 0.f, 0.f, 0x7FFFFFFF};
      if (valid && sp < g.splits) buf[i] = g.recs[static_cast<int64_t>(row) * g.splits + sp];
    }
    Rec r = buf[0];
#pragma unroll
    for (int i = 1; i < kFinRecs; ++i) rec_merge(r, buf[i], c);
    rec_merge(r, rec_dpp<kDppXor1>(r), c);
    rec_merge(r, rec_dpp<kDppXor2>(r), c);
    int keep_cat = 0;  // categorical: the row's drawn token (records merged in split order, then the quad)
    if (cat) {
      float bs = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int i = 0; i < kFinRecs; ++i) {
        const int sp = part + kFinParts * i;
        if (valid && sp < g.splits) {
          const GRec o = g.grecs[static_cast<int64_t>(row) * g.splits + sp];
          gmax(bs, bi, o.s, o.idx);
        }
      }
      gmax(bs, bi, dpp_f32<kDppXor1>(bs), static_cast<int>(dpp_u32<kDppXor1>(static_cast<uint32_t>(bi))));
      gmax(bs, bi, dpp_f32<kDppXor2>(bs), static_cast<int>(dpp_u32<kDppXor2>(static_cast<uint32_t>(bi))));
      keep_cat = bi;
    }
    if (valid && part == 0) {
      // The fold evaluates u = fma(l, c, -round(m c)): every u of a chunk carries the residual
      // delta = m c - round(m c); it cancels in H but not in ln Z.
      const float mc = r.m * c;
      const float delta = fmaf(r.m, c, -mc);
      const float lz = logf(r.z);
      const float H = lz - kLn2 * r.a / r.z;
      same &= g.pred[row] == r.idx ? 1 : 0;
      g.pred[row] = r.idx;
      const int keep = cat ? keep_cat : r.idx;  // the token an accepted position keeps
      if (group) {
        gH[row] = H;
        gIdx[row] = keep;
      } else {
        const bool acc = H <= g.bound;
        g.canvas[row] = acc ? keep : renoise_token(g, row);
        if (g.accept) g.accept[row] = acc ? 1 : 0;
      }
      if (g.entropy) g.entropy[row] = H;
      if (g.row_stats) {
        g.row_stats[2 * row] = r.m;
        g.row_stats[2 * row + 1] = lz - delta * kLn2;
      }
      hs += H;
    }
  }
  hs = wave_sum(hs);
  same = wave_min_i32(same);
  if (lane == 0) { shs[wave] = hs; shq[wave] = same; }
  __syncthreads();
  if (group) {
    // rank of each row in increasing (entropy, row) order; the rows' entropies in that order; one
    // thread walks the running total; rows ranked below the count are accepted
    int rk[kGroupMaxRows / kFinThreads];
#pragma unroll
    for (int i = 0; i < kGroupMaxRows / kFinThreads; ++i) {
      const int row = tid + i * kFinThreads;
      rk[i] = 0;
      if (row < g.rows) {
        const float h = gH[row];
        int n = 0;
        for (int j = 0; j < g.rows; ++j) {
          const float o = gH[j];
          n += (o < h || (o == h && j < row)) ? 1 : 0;
        }
        rk[i] = n;
      }
    }
    __syncthreads();  // every rank is computed before gH is overwritten in rank order
    float hv[kGroupMaxRows / kFinThreads];
#pragma unroll
    for (int i = 0; i < kGroupMaxRows / kFinThreads; ++i) {
      const int row = tid + i * kFinThreads;
      hv[i] = row < g.rows ? gH[row] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kGroupMaxRows / kFinThreads; ++i)
      if (tid + i * kFinThreads < g.rows) gH[rk[i]] = hv[i];
    __syncthreads();
    if (tid == 0) {
      float total = 0.f;
      int K = 0;
      for (int k = 0; k < g.rows; ++k) {
        total += gH[k];
        if (total > g.bound) break;
        K = k + 1;
      }
      gK = K;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kGroupMaxRows / kFinThreads; ++i) {
      const int row = tid + i * kFinThreads;
      if (row < g.rows) {
        const bool acc = rk[i] < gK;
        g.canvas[row] = acc ? gIdx[row] : renoise_token(g, row);
        if (g.accept) g.accept[row] = acc ? 1 : 0;
      }
    }
  }
  if (tid == 0) {
    float t = shs[0];
    int all = shq[0];
    for (int w = 1; w < kFinWaves; ++w) { t += shs[w]; all &= shq[w]; }
    const float meanH = t / static_cast<float>(g.rows);
    dg_stop_state st = *g.stop;
    st.stable_count = (g.step > 0 && all) ? st.stable_count + 1 : 0;
    st.mean_entropy = meanH;
    const bool confident = meanH < g.stop_thr, steady = st.stable_count >= g.stable_needed;
    st.stopped = ((g.mode & DG_SCHED_STOP_EITHER) ? (confident || steady) : (confident && steady)) ? 1 : 0;
    st.steps_run = g.step + 1;
    *g.stop = st;
  }
}

__global__ void init_canvas_kernel(uint64_t seed, int block, int n, uint32_t vocab, int32_t* __restrict__ canvas,
                                   dg_stop_state* __restrict__ stop) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) canvas[i] = draw_token(seed, static_cast<uint32_t>(i), 0u, static_cast<uint32_t>(block), kPurposeInit, vocab);
  if (i == 0 && stop != nullptr) {
    dg_stop_state st;
    st.mean_entropy = INFINITY;
    st.stable_count = 0;
    st.stopped = 0;
    st.steps_run = 0;
    *stop = st;
  }
}

// ----------------------------------------------------------------- host side
struct SplitPlan { int64_t splits, chunk; };

static SplitPlan plan_splits(int64_t rows, int64_t vocab) {
  const int64_t gran = kBatch;  // 8192 elements: whole batches
// workgroups a call aims at (16 per canvas row at 256 rows); measured on 256 x 262144 bf16 logits,
// 1024, 2048 and 8192 took 30.5, 29.3 and 35.4 us against 29.0
#ifndef DG_SAMP_WGS
#define DG_SAMP_WGS 4096
#endif
  const int64_t target_wgs = DG_SAMP_WGS;
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(ceil_div(vocab, gran), ceil_div(target_wgs, rows)));
  s = std::min<int64_t>(s, kMaxSplits);
  int64_t chunk = ceil_div(ceil_div(vocab, s), kVec) * kVec;
  if (chunk >= gran) chunk = ceil_div(chunk, gran) * gran;
  s = ceil_div(vocab, chunk);
  return {s, chunk};
}

static size_t recs_bytes(int64_t rows, int64_t vocab) {
  const SplitPlan p = plan_splits(rows, vocab);
  return (static_cast<size_t>(rows * p.splits) * sizeof(Rec) + 255) / 256 * 256;
}

size_t sample_fused_workspace_bytes(int64_t rows);

// the partial pass's records (and Gumbel records), or the merged records of the LM head's blocks
size_t sample_workspace_bytes(int64_t rows, int64_t vocab) {
  const SplitPlan p = plan_splits(rows, vocab);
  const size_t own = recs_bytes(rows, vocab) + (static_cast<size_t>(rows * p.splits) * sizeof(GRec) + 255) / 256 * 256;
  return std::max(own, sample_fused_workspace_bytes(rows));
}

int launch_init_canvas(uint64_t seed, int block, int n, int vocab, int32_t* canvas, dg_stop_state* stop,
                       hipStream_t stream) {
  const int threads = 256;
  const int grid = std::max(1, static_cast<int>(ceil_div(n, threads)));
  ProfScope ps("init_canvas", stream);
  init_canvas_kernel<<<grid, threads, 0, stream>>>(seed, block, n, static_cast<uint32_t>(vocab), canvas, stop);
  DG_LAUNCH_CHECK("init_canvas_kernel");
  return DG_OK;
}

// ------------------------------------------------ static scratch (no allocation)
// The partial records of dg_sample_canvas_static live here instead of in a caller workspace. In host
// code `scratch` names a host-side stand-in, never the device array: the device address is taken
// once per device with hipGetSymbolAddress (that device current) and used from then on. Every call on
// one device shares that device's array; the partial kernel writes every record the finalize kernel
// reads, so nothing in it has to start at zero, but calls that overlap in time on one device race.
constexpr size_t kStaticScratchBytes = size_t{1} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// device address of this device's scratch (looked up on the first call per device)
int static_scratch(void** out) {
  int dev = 0;
  DG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    DG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(DG_ERR_HIP, "hipGetSymbolAddress returned no address for the sampler scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

int launch_sample(const void* logits, int dtype, int rows, int vocab, float temp, const dg_sched& sc, int step,
                  int block, int32_t* canvas, int32_t* pred, uint8_t* accept, float* entropy, float* row_stats,
                  dg_stop_state* stop, void* ws, hipStream_t stream) {
  const SplitPlan p = plan_splits(rows, vocab);
  SampleArgs g;
  g.logits = logits;
  g.vocab = vocab;
  g.chunk = p.chunk;
  g.rows = rows;
  g.splits = static_cast<int>(p.splits);
  g.c = kLog2e / temp;
  g.bound = sc.entropy_bound;
  g.stop_thr = sc.stop_mean_entropy;
  g.stable_needed = sc.stable_needed;
  g.mode = sc.mode;
  if ((sc.mode & DG_SCHED_ACCEPT_GROUP) && rows > kGroupMaxRows)
    return fail(DG_ERR_UNSUPPORTED, "group acceptance: at most 4096 rows");
  if ((sc.mode & DG_SCHED_SAMPLE) && vocab % kVec != 0)
    return fail(DG_ERR_UNSUPPORTED, "categorical sampling: vocab must be a multiple of 8");
  g.seed = sc.seed;
  g.step = step;
  g.block = block;
  g.canvas = canvas; g.pred = pred; g.accept = accept; g.entropy = entropy; g.row_stats = row_stats; g.stop = stop;
  g.recs = static_cast<Rec*>(ws);
  g.grecs = reinterpret_cast<GRec*>(static_cast<char*>(ws) + recs_bytes(rows, vocab));
  g.inv_t = 1.0f / temp;
  dim3 grid(static_cast<unsigned>(p.splits), static_cast<unsigned>(rows));
  {
    ProfScope ps("sample_partial", stream);
    const bool vec = vocab % kVec == 0;
    const bool cat = (sc.mode & DG_SCHED_SAMPLE) != 0;
    const dim3 block(kSampThreads);
    if (dtype == DG_BF16) {
      if (cat) sample_kernel<bf16_t, true, true><<<grid, block, 0, stream>>>(g);
      else if (vec) sample_kernel<bf16_t, true, false><<<grid, block, 0, stream>>>(g);
      else sample_kernel<bf16_t, false, false><<<grid, block, 0, stream>>>(g);
    } else {
      if (cat) sample_kernel<float, true, true><<<grid, block, 0, stream>>>(g);
      else if (vec) sample_kernel<float, true, false><<<grid, block, 0, stream>>>(g);
      else sample_kernel<float, false, false><<<grid, block, 0, stream>>>(g);
    }
  }
  DG_LAUNCH_CHECK("sample_kernel");
  {
    ProfScope ps("sample_finalize", stream);
    sample_finalize_kernel<<<1, kFinThreads, 0, stream>>>(g);
  }
  DG_LAUNCH_CHECK("sample_finalize_kernel");
  return DG_OK;
}

// ------------------------------------------------ records produced by the LM head
// The LM head can fold its own output into split-row records, one per (row, 256-column vocabulary
// block), in the same layout and arithmetic as the partial pass (vocab.hip). The records of a row
// are merged here into kFusedSplits records, one wave per (row, run of consecutive blocks) in a
// fixed order, and the finalize kernel runs on those as on the partial pass's: the logits are not
// read again.
constexpr int kFusedSplits = 16;

__global__ __launch_bounds__(256) void merge_block_recs_kernel(SampleArgs g, const Rec* __restrict__ brec, int nblk) {
  if (g.stop->stopped) return;
  const int lane = threadIdx.x & 63;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, group)
  const int row = wv / kFusedSplits, grp = wv - row * kFusedSplits;
  if (row >= g.rows) return;
  const int per = (nblk + kFusedSplits - 1) / kFusedSplits;
  const int b0 = grp * per, b1 = min(nblk, b0 + per);
  Rec r{-INFINITY, 0.f, 0.f, 0x7FFFFFFF};
  for (int b = b0 + lane; b < b1; b += 64) rec_merge(r, brec[static_cast<int64_t>(row) * nblk + b], g.c);
  rec_wave_merge(r, g.c);
  if (lane == 0) g.recs[static_cast<int64_t>(row) * kFusedSplits + grp] = r;
}

size_t sample_fused_workspace_bytes(int64_t rows) {
  return (static_cast<size_t>(rows * kFusedSplits) * sizeof(Rec) + 255) / 256 * 256;
}

int launch_sample_from_block_recs(const void* block_recs, int nblk, int rows, int vocab, float temp,
                                  const dg_sched& sc, int step, int block, int32_t* canvas, int32_t* pred,
                                  uint8_t* accept, float* entropy, float* row_stats, dg_stop_state* stop, void* ws,
                                  hipStream_t stream) {
  if (sc.mode & DG_SCHED_SAMPLE)
    return fail(DG_ERR_UNSUPPORTED, "records from the LM head: categorical sampling needs the partial pass");
  if ((sc.mode & DG_SCHED_ACCEPT_GROUP) && rows > kGroupMaxRows)
    return fail(DG_ERR_UNSUPPORTED, "group acceptance: at most 4096 rows");
  if (nblk < 1) return fail(DG_ERR_INVALID, "no LM head records");
  SampleArgs g;
  g.logits = nullptr;
  g.vocab = vocab;
  g.chunk = vocab;
  g.rows = rows;
  g.splits = kFusedSplits;
  g.c = kLog2e / temp;
  g.bound = sc.entropy_bound;
  g.stop_thr = sc.stop_mean_entropy;
  g.stable_needed = sc.stable_needed;
  g.mode = sc.mode;
  g.seed = sc.seed;
  g.step = step;
  g.block = block;
  g.canvas = canvas; g.pred = pred; g.accept = accept; g.entropy = entropy; g.row_stats = row_stats; g.stop = stop;
  g.recs = static_cast<Rec*>(ws);
  g.grecs = nullptr;
  g.inv_t = 1.0f / temp;
  {
    ProfScope ps("sample_merge", stream);
    const int waves = rows * kFusedSplits;
    merge_block_recs_kernel<<<(waves + 3) / 4, 256, 0, stream>>>(g, static_cast<const Rec*>(block_recs), nblk);
  }
  DG_LAUNCH_CHECK("merge_block_recs_kernel");
  {
    ProfScope ps("sample_finalize", stream);
    sample_finalize_kernel<<<1, kFinThreads, 0, stream>>>(g);
  }
  DG_LAUNCH_CHECK("sample_finalize_kernel");
  return DG_OK;
}

}  // namespace dg
