// Attention of a chunk of M query rows over the KV cache, grouped-query.
//
// Denoiser mode is bidirectional: every canvas query sees all cached
// positions and every canvas position ([P3] "Encoder-denoiser design":
// causal attention becomes bidirectional over the whole noisy canvas).
// Encoder mode (prompt prefill, block commit) is causal ([P3] same section:
// the query is processed the standard way). Scores are scaled by
// 1/sqrt(head_dim); query head j reads KV head floor(j * Hkv / Hq).
//
// bf16 path (MFMA, split-KV flash attention). A workgroup owns 64 query rows
// of one KV-head group (the Hq/Hkv query heads sharing that KV head are laid
// side by side, so a K/V tile serves all of them) and one slice of the keys;
// each of its 4 waves owns one 16-query tile (kQT; two tiles per wave double
// the register footprint and halve occupancy). K and V^T tiles of
// 64 keys are staged through LDS, and the next tile is already being fetched
// into registers while the current one is multiplied. Each wave works on the
// transposed scores S^T = K Q^T: in the 16x16 accumulator layout every lane
// then owns a single query column, so the online-softmax state (running max
// and sum) is per lane and the rescale of O^T is a per-lane multiply. The
// probabilities already sit in the lane/k arrangement the second MFMA wants
// for P^T as its B operand (lane group g holds keys 4g..4g+3 of two adjacent
// 16-key tiles, a permutation of the 32 keys of the k-step), and V^T is read
// from LDS with the same key permutation, so P never goes through LDS.
// Each workgroup writes (max, sum, unnormalised O) for its key slice; a merge
// kernel (one wave per query row) combines the slices in a fixed order.
// Exponentials are base 2 with log2(e) folded into the scale.
//
// fp32 path: a direct kernel, one thread per (query row, head), online
// softmax over all keys; used for the small fp32 configuration.
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "mfma.h"
#include "prof.h"

namespace dg {

struct AttnArgs {
  const void* q;        // [M x Hq*hd]
  int64_t ldq;
  const void* kc;       // [Hkv][cap][hd] of this layer
  const void* vc;
  int64_t head_stride;  // cap * hd
  int M, Hq, Hkv, hd;
  int pos0;             // absolute position of query row 0; keys 0 .. pos0+M-1
  int causal;
  float scale_log2;     // log2(e) / sqrt(hd)
  int splits;
  int key_chunk;        // keys per split (multiple of 64)
  float* part_o;        // [splits][Hq*M][hd]
  float* part_ml;       // [splits][Hq*M][2]
  void* o;              // [M x Hq*hd] output (merge)
  int64_t ldo;
};

constexpr int kKB = 64;                    // keys per LDS block
constexpr int kQT = 1;                     // 16-query tiles per wave
constexpr int kWGRows = 4 * kQT * 16;      // query rows per workgroup

template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KPAD = HD + 8;    // sK row pitch (bf16)
  constexpr int VPAD = kKB + 8;   // sVt row pitch (bf16)
  constexpr int HS = HD / 32;     // k-steps over head_dim
  constexpr int HT = HD / 16;     // O^T tiles over head_dim
  constexpr int CH = HD / 8;      // 16-byte chunks per key row
  constexpr int LOADS = kKB * CH / 256;
  __shared__ __align__(16) bf16_t sK[kKB * KPAD];
  __shared__ __align__(16) bf16_t sVt[HD * VPAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int rows_in_group = G * a.M;
  const int kvh = blockIdx.y;
  const int split = blockIdx.z;
  const int L = a.pos0 + a.M;
  const int g4 = lane >> 4;

  int qr[kQT], qhead[kQT], qm[kQT], qpos[kQT];
  bool qvalid[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    qr[t] = blockIdx.x * kWGRows + (wave * kQT + t) * 16 + (lane & 15);
    qvalid[t] = qr[t] < rows_in_group;
    qhead[t] = kvh * G + (qvalid[t] ? qr[t] / a.M : 0);
    qm[t] = qvalid[t] ? qr[t] % a.M : 0;
    qpos[t] = a.pos0 + qm[t];
  }

  // key range of this split, clipped for causal attention to the workgroup's last position
  const int k_lo = split * a.key_chunk;
  int k_hi = min(L, k_lo + a.key_chunk);
  if (a.causal) {
    const int first_row = blockIdx.x * kWGRows;
    const int last_row = min(rows_in_group - 1, first_row + kWGRows - 1);
    int maxpos = a.pos0 + a.M - 1;
    if (first_row / a.M == last_row / a.M) maxpos = a.pos0 + last_row % a.M;
    k_hi = min(k_hi, maxpos + 1);
  }

  // Q^T fragments (B operand): lane supplies query qr, head dims 8*g4 .. of each 32-step
  bf16x8_t qf[kQT][HS];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qm[t]) * a.ldq + qhead[t] * HD;
#pragma unroll
    for (int h = 0; h < HS; ++h) qf[t][h] = qvalid[t] ? Frag<bf16_t>::load(qb + h * 32 + g4 * 8) : Frag<bf16_t>::zero();
  }

  f32x4_t o[kQT][HT];
  float mrun[kQT], lrun[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
#pragma unroll
    for (int j = 0; j < HT; ++j) o[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mrun[t] = -INFINITY;
    lrun[t] = 0.f;
  }

  const bf16_t* kbase = static_cast<const bf16_t*>(a.kc) + kvh * a.head_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.vc) + kvh * a.head_stride;
  uint4 pk[LOADS], pv[LOADS];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int key = c / CH, ch = c % CH;
      pk[i] = make_uint4(0, 0, 0, 0);
      pv[i] = make_uint4(0, 0, 0, 0);
      if (kb + key < k_hi) {
        pk[i] = *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(kb + key) * HD + ch * 8);
        pv[i] = *reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(kb + key) * HD + ch * 8);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int key = c / CH, ch = c % CH;
      *reinterpret_cast<uint4*>(&sK[key * KPAD + ch * 8]) = pk[i];
      const uint32_t w[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(ch * 8 + 2 * e) * VPAD + key] = static_cast<bf16_t>(w[e] & 0xFFFF);
        sVt[(ch * 8 + 2 * e + 1) * VPAD + key] = static_cast<bf16_t>(w[e] >> 16);
      }
    }
  };

  if (k_lo < k_hi) gload(k_lo);
  for (int kb = k_lo; kb < k_hi; kb += kKB) {
    __syncthreads();  // every wave is done with the previous block
    sstore();
    __syncthreads();
    if (kb + kKB < k_hi) gload(kb + kKB);  // next block in flight during this one

#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      // ---- S^T = K Q^T for 4 key tiles of 16
      f32x4_t s[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HS; ++h) {
          const bf16x8_t kf = Frag<bf16_t>::load(&sK[(kt * 16 + (lane & 15)) * KPAD + h * 32 + g4 * 8]);
          acc = Frag<bf16_t>::mma(kf, qf[t][h], acc);
        }
        s[kt] = acc;
      }
      // scale, mask, block max (this lane's 16 keys, then the 4 lane groups)
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + kt * 16 + g4 * 4 + i;
          float v = s[kt][i] * a.scale_log2;
          const bool ok = key < k_hi && (!a.causal || key <= qpos[t]);
          v = ok ? v : -INFINITY;
          s[kt][i] = v;
          bmax = fmaxf(bmax, v);
        }
      bmax = fmaxf(bmax, shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, shfl_xor(bmax, 32));
      const float mnew = fmaxf(mrun[t], bmax);
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // all masked so far: keep the base finite
      const float alpha = exp2f(mrun[t] - mref);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(s[kt][i] - mref);
          s[kt][i] = p;
          psum += p;
        }
      psum += shfl_xor(psum, 16);
      psum += shfl_xor(psum, 32);
      lrun[t] = lrun[t] * alpha + psum;
      mrun[t] = mnew;
#pragma unroll
      for (int j = 0; j < HT; ++j) o[t][j] *= alpha;

      // ---- O^T += V^T P^T, two k-steps of 32 keys
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t pf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[i] = static_cast<__bf16>(s[2 * ks][i]);
          pf[4 + i] = static_cast<__bf16>(s[2 * ks + 1][i]);
        }
#pragma unroll
        for (int j = 0; j < HT; ++j) {
          const bf16_t* vr = &sVt[(j * 16 + (lane & 15)) * VPAD + ks * 32 + g4 * 4];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
          bf16x8_t vf;
          const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
          __builtin_memcpy(&vf, w, 16);
          o[t][j] = Frag<bf16_t>::mma(vf, pf, o[t][j]);
        }
      }
    }
  }

  // ---- partial results: lane holds O^T[hd = j*16 + 4*g4 + i][query qr]
  const int64_t R = static_cast<int64_t>(a.Hq) * a.M;
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    if (!qvalid[t]) continue;
    const int64_t row = static_cast<int64_t>(qhead[t]) * a.M + qm[t];
    float* po = a.part_o + (split * R + row) * HD;
#pragma unroll
    for (int j = 0; j < HT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[j * 16 + g4 * 4 + i] = o[t][j][i];
    if (g4 == 0) {
      a.part_ml[(split * R + row) * 2] = mrun[t];
      a.part_ml[(split * R + row) * 2 + 1] = lrun[t];
    }
  }
}

// combine the key slices, one wave per query row:
// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int hd) {
  const int64_t R = static_cast<int64_t>(a.Hq) * a.M;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  float ms = -INFINITY, ls = 0.f;
  if (lane < a.splits) {
    ms = a.part_ml[(lane * R + row) * 2];
    ls = a.part_ml[(lane * R + row) * 2 + 1];
  }
  const float mx = wave_max(ms);
  const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
  const float l = wave_sum(w * ls);
  const int head = static_cast<int>(row / a.M), m = static_cast<int>(row % a.M);
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ws = __shfl(w, s, 64);
      if (ws != 0.f) acc += ws * a.part_o[(s * R + row) * hd + d];
    }
    const float v = l > 0.f ? acc / l : 0.f;
    static_cast<T*>(a.o)[static_cast<int64_t>(m) * a.ldo + head * hd + d] = from_f32<T>(v);
  }
}

// fp32: one thread per (query row, head)
__global__ void attn_f32_kernel(AttnArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * a.Hq) return;
  const int m = idx / a.Hq, j = idx % a.Hq;
  const int kvh = (j * a.Hkv) / a.Hq;
  const int hd = a.hd;
  const float* q = static_cast<const float*>(a.q) + static_cast<int64_t>(m) * a.ldq + j * hd;
  const float* kb = static_cast<const float*>(a.kc) + kvh * a.head_stride;
  const float* vb = static_cast<const float*>(a.vc) + kvh * a.head_stride;
  const int L = a.causal ? a.pos0 + m + 1 : a.pos0 + a.M;
  float acc[128];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  float mx = -INFINITY, l = 0.f;
  for (int t = 0; t < L; ++t) {
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += q[d] * kb[static_cast<int64_t>(t) * hd + d];
    s *= a.scale_log2;
    const float mn = fmaxf(mx, s);
    const float al = exp2f(mx - mn), p = exp2f(s - mn);
    l = l * al + p;
    for (int d = 0; d < hd; ++d) acc[d] = acc[d] * al + p * vb[static_cast<int64_t>(t) * hd + d];
    mx = mn;
  }
  float* o = static_cast<float*>(a.o) + static_cast<int64_t>(m) * a.ldo + j * hd;
  for (int d = 0; d < hd; ++d) o[d] = acc[d] / l;
}

// ------------------------------------------------------------------- host
int attn_max_splits() { return 32; }

int attention(const void* q, int64_t ldq, const void* kc, const void* vc, int64_t head_stride, int M, int Hq,
              int Hkv, int hd, int pos0, int causal, float* part_o, float* part_ml, void* o, int64_t ldo,
              int dtype, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.kc = kc; a.vc = vc; a.head_stride = head_stride;
  a.M = M; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.pos0 = pos0; a.causal = causal;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(hd)));
  a.part_o = part_o; a.part_ml = part_ml; a.o = o; a.ldo = ldo;
  const int L = pos0 + M;
  if (dtype == DG_F32) {
    if (hd > 128) return fail(DG_ERR_UNSUPPORTED, "fp32 attention needs head_dim <= 128");
    a.splits = 1;
    ProfScope ps("attention_f32", s);
    const int n = M * Hq;
    attn_f32_kernel<<<(n + 127) / 128, 128, 0, s>>>(a);
    DG_LAUNCH_CHECK("attn_f32_kernel");
    return DG_OK;
  }
  if (hd != 64 && hd != 128) return fail(DG_ERR_UNSUPPORTED, "bf16 attention needs head_dim 64 or 128");
  const int G = Hq / Hkv;
  const int qtiles = (G * M + kWGRows - 1) / kWGRows;
  // about 512 workgroups, at least two key blocks per split
  int splits = std::max(1, std::min(attn_max_splits(), (512 + qtiles * Hkv - 1) / (qtiles * Hkv)));
  splits = std::min(splits, std::max(1, (L + 2 * kKB - 1) / (2 * kKB)));
  a.key_chunk = ((L + splits - 1) / splits + kKB - 1) / kKB * kKB;
  a.splits = (L + a.key_chunk - 1) / a.key_chunk;
  dim3 grid(qtiles, Hkv, a.splits);
  {
    ProfScope ps("attention", s);
    if (hd == 128) attn_bf16_kernel<128><<<grid, 256, 0, s>>>(a);
    else attn_bf16_kernel<64><<<grid, 256, 0, s>>>(a);
  }
  DG_LAUNCH_CHECK("attn_bf16_kernel");
  {
    ProfScope ps("attention_merge", s);
    const int64_t rows = static_cast<int64_t>(Hq) * M;
    attn_merge_kernel<bf16_t><<<static_cast<int>((rows + 3) / 4), 256, 0, s>>>(a, hd);
  }
  DG_LAUNCH_CHECK("attn_merge_kernel");
  return DG_OK;
}

}  // namespace dg
