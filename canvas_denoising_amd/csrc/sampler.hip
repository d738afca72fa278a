// Entropy-bounded sampler over the canvas logits, one read of the logits.
//
// [P3] "Inference mechanism": the logits scheduler sharpens with a
// temperature; the entropy-bounded sampler accepts tokens by an entropy-based
// confidence and re-noises the others with random tokens. [P4] "Standard
// sampling settings" (table) and "Two-Fold Adaptive Stopping" give the
// constants and the stop rule.
//
// Split-row design: a [rows x vocab] logits matrix has far too few rows for
// 256 CUs, so every row is cut into `splits` chunks. One workgroup streams
// one chunk once (16-byte coalesced loads) and reduces it to a record
// (m = max logit, Z = sum 2^u, A = sum u 2^u with u = (l - m) * log2(e) / T,
// argmax index). Records merge exactly:
//   m = max(m1, m2), d_i = (m_i - m) log2(e)/T,
//   Z = Z1 2^d1 + Z2 2^d2,  A = 2^d1 (A1 + d1 Z1) + 2^d2 (A2 + d2 Z2),
// so the finalize pass gets the row entropy H = ln Z - ln2 * A / Z without
// a second read. The finalize kernel merges the records of each row in a
// fixed order, applies the accept / re-noise rule with Philox, and reduces
// the canvas mean entropy and the stop state in a fixed order (results are
// bitwise reproducible).
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "philox.h"
#include "prof.h"

namespace dg {

struct Rec {
  float m;   // max raw logit (-inf when empty)
  float z;   // sum 2^u
  float a;   // sum u 2^u
  int idx;   // lowest index attaining m
};

__device__ inline void rec_merge(Rec& x, const Rec& y, float c) {
  if (y.z == 0.f) return;
  if (x.z == 0.f) { x = y; return; }
  const float m = fmaxf(x.m, y.m);
  const float dx = (x.m - m) * c, dy = (y.m - m) * c;
  const float sx = exp2f(dx), sy = exp2f(dy);
  const int idx = (x.m > y.m) ? x.idx : (y.m > x.m) ? y.idx : min(x.idx, y.idx);
  x.a = sx * (x.a + dx * x.z) + sy * (y.a + dy * y.z);
  x.z = x.z * sx + y.z * sy;
  x.m = m;
  x.idx = idx;
}

__device__ inline Rec rec_shfl_xor(const Rec& r, int mask) {
  Rec o;
  o.m = shfl_xor(r.m, mask);
  o.z = shfl_xor(r.z, mask);
  o.a = shfl_xor(r.a, mask);
  o.idx = shfl_xor(r.idx, mask);
  return o;
}

// 8 consecutive logits as fp32
template <typename T> struct Load8;
template <> struct Load8<bf16_t> {
  __device__ static inline void run(const bf16_t* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
    v[4] = bf16lo(q.z); v[5] = bf16hi(q.z); v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
  }
};
template <> struct Load8<float> {
  __device__ static inline void run(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T> __device__ inline float load1(const T* p);
template <> __device__ inline float load1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <> __device__ inline float load1<float>(const float* p) { return *p; }

constexpr int kSampThreads = 256;
constexpr int kVec = 8;      // elements per vector load
constexpr int kUnroll = 4;   // vector loads per thread per batch
constexpr int kBatch = kSampThreads * kVec * kUnroll;  // elements per workgroup batch

// Accumulate N fp32 values into the running record. Value j sits at logit index
// idx0 + (j / 8) * gstride + (j % 8); within the thread indices grow with j, so
// the first strictly larger value is the lowest index of the batch maximum.
template <int N>
__device__ inline void accumulate(const float* v, int64_t idx0, int64_t gstride, float c, Rec& r) {
  float bm = v[0];
  int bk = 0;
#pragma unroll
  for (int j = 1; j < N; ++j) {
    if (v[j] > bm) { bm = v[j]; bk = j; }
  }
  if (bm > r.m) {  // new running max: rescale what was accumulated so far
    if (r.z != 0.f) {
      const float d = (r.m - bm) * c;
      const float s = exp2f(d);
      r.a = s * (r.a + d * r.z);
      r.z *= s;
    }
    r.m = bm;
    r.idx = static_cast<int>(idx0 + (bk >> 3) * gstride + (bk & 7));
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
}

// grid (splits, rows); each workgroup reduces logits[row, sp*chunk : (sp+1)*chunk)
template <typename T, bool kVecPath>
__global__ __launch_bounds__(kSampThreads) void sample_partial_kernel(
    const T* __restrict__ logits, int64_t vocab, int64_t chunk, float c,
    const dg_stop_state* __restrict__ stop, Rec* __restrict__ recs) {
  if (stop != nullptr && stop->stopped) return;
  const int sp = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int64_t begin = sp * chunk;
  const int64_t end = min(begin + chunk, vocab);
  const T* p = logits + static_cast<int64_t>(row) * vocab;
  Rec r{-INFINITY, 0.f, 0.f, 0x7FFFFFFF};

  if (kVecPath) {
    // full batches: every thread owns kUnroll groups of 8 consecutive elements
    int64_t base = begin;
    for (; base + kBatch <= end; base += kBatch) {
      float v[kUnroll * kVec];
      const int64_t t0 = base + static_cast<int64_t>(tid) * kVec;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) Load8<T>::run(p + t0 + static_cast<int64_t>(u) * kSampThreads * kVec, v + u * kVec);
      accumulate<kUnroll * kVec>(v, t0, static_cast<int64_t>(kSampThreads) * kVec, c, r);
    }
    // tail: whole groups of 8 (vocab % 8 == 0 on this path)
    for (int64_t e0 = base + static_cast<int64_t>(tid) * kVec; e0 < end; e0 += static_cast<int64_t>(kSampThreads) * kVec) {
      float v[kVec];
      Load8<T>::run(p + e0, v);
      accumulate<kVec>(v, e0, 0, c, r);
    }
  } else {
    for (int64_t e = begin + tid; e < end; e += kSampThreads) {
      float v[1] = {load1<T>(p + e)};
      accumulate<1>(v, e, 0, c, r);
    }
  }

  // wave then workgroup reduction (fixed butterfly / fixed wave order)
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const Rec o = rec_shfl_xor(r, m);
    rec_merge(r, o, c);
  }
  __shared__ Rec sh[kSampThreads / 64];
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) sh[wave] = r;
  __syncthreads();
  if (tid == 0) {
    Rec acc = sh[0];
    for (int w = 1; w < kSampThreads / 64; ++w) rec_merge(acc, sh[w], c);
    recs[static_cast<int64_t>(row) * gridDim.x + sp] = acc;
  }
}

constexpr int kFinThreads = 256;

// one workgroup: merge split records per row, accept / re-noise, canvas stats, stop rule
__global__ __launch_bounds__(kFinThreads) void sample_finalize_kernel(
    const Rec* __restrict__ recs, int rows, int splits, float c, float inv_temp,
    float bound, float stop_thr, int stable_needed, uint64_t seed, int step, int block, uint32_t vocab,
    int32_t* __restrict__ canvas, int32_t* __restrict__ pred, uint8_t* __restrict__ accept,
    float* __restrict__ entropy, float* __restrict__ row_stats, dg_stop_state* __restrict__ stop) {
  if (stop != nullptr && stop->stopped) return;
  const int tid = threadIdx.x;
  float hsum = 0.f;
  int same = 1;
  for (int row = tid; row < rows; row += kFinThreads) {
    Rec r = recs[static_cast<int64_t>(row) * splits];
    for (int s = 1; s < splits; ++s) rec_merge(r, recs[static_cast<int64_t>(row) * splits + s], c);
    const float lnz = logf(r.z);
    const float H = lnz - kLn2 * r.a / r.z;
    const bool acc = H <= bound;
    const int32_t prv = pred[row];
    same &= (prv == r.idx) ? 1 : 0;
    pred[row] = r.idx;
    canvas[row] = acc ? r.idx
                      : draw_token(seed, static_cast<uint32_t>(row), static_cast<uint32_t>(step),
                                   static_cast<uint32_t>(block), kPurposeRenoise, vocab);
    if (accept) accept[row] = acc ? 1 : 0;
    if (entropy) entropy[row] = H;
    if (row_stats) {
      row_stats[2 * row] = r.m;
      row_stats[2 * row + 1] = lnz;
    }
    hsum += H;
  }
  (void)inv_temp;
  hsum = wave_sum(hsum);
  // wave-wide AND of `same`
  for (int m = 32; m >= 1; m >>= 1) same &= shfl_xor(same, m);
  __shared__ float shs[kFinThreads / 64];
  __shared__ int shq[kFinThreads / 64];
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) { shs[wave] = hsum; shq[wave] = same; }
  __syncthreads();
  if (tid == 0) {
    float tot = shs[0];
    int all = shq[0];
    for (int w = 1; w < kFinThreads / 64; ++w) { tot += shs[w]; all &= shq[w]; }
    const float meanH = tot / static_cast<float>(rows);
    dg_stop_state st = *stop;
    st.stable_count = (step > 0 && all) ? st.stable_count + 1 : 0;
    st.mean_entropy = meanH;
    st.stopped = (meanH < stop_thr && st.stable_count >= stable_needed) ? 1 : 0;
    st.steps_run = step + 1;
    *stop = st;
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
  const int64_t gran = kSampThreads * kVec;  // 2048
  const int64_t target_wgs = 4096;
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(ceil_div(vocab, gran), ceil_div(target_wgs, rows)));
  int64_t chunk = ceil_div(ceil_div(vocab, s), gran) * gran;
  s = ceil_div(vocab, chunk);
  return {s, chunk};
}

size_t sample_workspace_bytes(int64_t rows, int64_t vocab) {
  const SplitPlan p = plan_splits(rows, vocab);
  return static_cast<size_t>(rows * p.splits) * sizeof(Rec);
}

int launch_init_canvas(uint64_t seed, int block, int n, int vocab, int32_t* canvas, dg_stop_state* stop,
                       hipStream_t stream) {
  const int threads = 256;
  const int grid = std::max(1, static_cast<int>(ceil_div(n, threads)));
  init_canvas_kernel<<<grid, threads, 0, stream>>>(seed, block, n, static_cast<uint32_t>(vocab), canvas, stop);
  DG_LAUNCH_CHECK("init_canvas_kernel");
  return DG_OK;
}

int launch_sample(const void* logits, int dtype, int rows, int vocab, float temp, const dg_sched& sc, int step,
                  int block, int32_t* canvas, int32_t* pred, uint8_t* accept, float* entropy, float* row_stats,
                  dg_stop_state* stop, void* ws, hipStream_t stream) {
  const SplitPlan p = plan_splits(rows, vocab);
  const float c = kLog2e / temp;
  Rec* recs = static_cast<Rec*>(ws);
  dim3 grid(static_cast<unsigned>(p.splits), static_cast<unsigned>(rows));
  {
  ProfScope ps("sample_partial", stream);
  if (dtype == DG_BF16) {
    const bf16_t* l = static_cast<const bf16_t*>(logits);
    if (vocab % kVec == 0)
      sample_partial_kernel<bf16_t, true><<<grid, kSampThreads, 0, stream>>>(l, vocab, p.chunk, c, stop, recs);
    else
      sample_partial_kernel<bf16_t, false><<<grid, kSampThreads, 0, stream>>>(l, vocab, p.chunk, c, stop, recs);
  } else {
    const float* l = static_cast<const float*>(logits);
    if (vocab % kVec == 0)
      sample_partial_kernel<float, true><<<grid, kSampThreads, 0, stream>>>(l, vocab, p.chunk, c, stop, recs);
    else
      sample_partial_kernel<float, false><<<grid, kSampThreads, 0, stream>>>(l, vocab, p.chunk, c, stop, recs);
  }
  }
  DG_LAUNCH_CHECK("sample_partial_kernel");
  {
  ProfScope ps("sample_finalize", stream);
  sample_finalize_kernel<<<1, kFinThreads, 0, stream>>>(
      recs, rows, static_cast<int>(p.splits), c, 1.0f / temp, sc.entropy_bound, sc.stop_mean_entropy,
      sc.stable_needed, sc.seed, step, block, static_cast<uint32_t>(vocab), canvas, pred, accept, entropy,
      row_stats, stop);
  }
  DG_LAUNCH_CHECK("sample_finalize_kernel");
  return DG_OK;
}

}  // namespace dg
