// Attention of a chunk of M query rows over the KV cache, grouped-query.
//
// Denoiser mode is bidirectional: every canvas query sees all cached
// positions and every canvas position ([P3] "Encoder-denoiser design":
// causal attention becomes bidirectional over the whole noisy canvas).
// Encoder mode (prompt prefill, block commit) is causal ([P3] same section:
// the query is processed the standard way). Scores are scaled by
// 1/sqrt(head_dim); query head j reads KV head floor(j * Hkv / Hq).
//
// bf16 path (MFMA, split-KV flash attention). A workgroup of 8 waves owns
// the query rows of one KV-head group (the Hq/Hkv query heads sharing that KV
// head are laid side by side, so one K/V tile serves all of them) and one
// slice of the keys; each wave owns one 16-query tile in canvas passes and
// two in longer passes (prefill chunks), where every K and V fragment read
// from LDS then feeds two MFMAs. K and V^T tiles stream into a ring of LDS
// stages by asynchronous global->LDS copies (dma.h), one barrier per stage:
// 128 keys in a ring of 2 for canvas passes, 64 keys in a ring of 3 for the
// longer ones. The V cache is stored transposed in 32-position blocks
// (kvlayout.h), so a V^T stage is one contiguous copy and each V^T fragment
// one 16-byte LDS read per lane; K rows are XOR-swizzled in LDS so the 16
// rows a fragment read touches fall on distinct banks. Each wave works on the
// transposed scores S^T = K Q^T: in the 16x16 accumulator layout every lane
// then owns a single query column, so the online-softmax state (running max
// and sum) is per lane and the rescale of O^T is a per-lane multiply. The
// probabilities already sit in the lane/k arrangement the second MFMA wants
// for P^T as its B operand (lane group g holds keys 4g..4g+3 of both 16-key
// tiles), which is the slot order of the V cache blocks, so P never goes
// through LDS. Each workgroup writes (max, sum, unnormalised O) for its key
// slice and a merge kernel (one wave per query row) combines the slices in a
// fixed order; with a single slice the kernel writes O itself.
// Exponentials are base 2 with log2(e) folded into the scale.
//
// fp32 path: a direct kernel, one thread per (query row, head), online
// softmax over all keys; used for the small fp32 configuration.
#include <math.h>

#include <algorithm>

#include "dg_common.h"
#include "mfma.h"
#include "dma.h"
#include "kvlayout.h"
#include "prof.h"

namespace dg {

struct AttnArgs {
  const void* q;        // [M x Hq*hd]
  int64_t ldq;
  const void* kc;       // K [Hkv][cap][hd] of this layer
  const void* vc;       // V [Hkv][cap/32][hd][32] (kvlayout.h)
  int64_t head_stride;  // cap * hd
  int M, Hq, Hkv, hd;
  int pos0;             // absolute position of query row 0; keys 0 .. pos0+M-1
  const int* pos_dev;   // when set, pos0 is *pos_dev (read on the device) and key_chunk follows from it
  int causal;
  float scale_log2;     // log2(e) / sqrt(hd)
  int splits;
  int qtiles;           // query-row tiles of kWGRows per KV-head group
  int key_chunk;        // keys per split (multiple of 32)
  float* part_o;        // [splits][Hq*M][hd]
  float* part_ml;       // [splits][Hq*M][2]
  void* o;              // [M x Hq*hd] output (merge)
  int64_t ldo;
};

// Stage shape: V blocks per LDS stage (KB2, 32 keys each) and ring depth (NS, NS - 1 stages in
// flight). Canvas passes (one query tile per wave) take 128-key stages in a ring of 2: half the
// barriers of 64-key stages for the same bytes in flight. Passes with two query tiles per wave
// (prefill chunks) keep 64-key stages in a ring of 3, whose fragments fit their registers.
#ifndef DG_ATT_KB2
#define DG_ATT_KB2 4
#endif
#ifndef DG_ATT_NS
#define DG_ATT_NS 2
#endif
#ifndef DG_ATT_KB2_LARGE
#define DG_ATT_KB2_LARGE 2
#endif
#ifndef DG_ATT_NS_LARGE
#define DG_ATT_NS_LARGE 3
#endif
constexpr int kVB = 32;  // positions per V cache block (kvlayout.h)
__host__ __device__ constexpr int att_kb2(int qt) { return qt == 1 ? DG_ATT_KB2 : DG_ATT_KB2_LARGE; }
__host__ __device__ constexpr int att_stages(int qt) { return qt == 1 ? DG_ATT_NS : DG_ATT_NS_LARGE; }
__host__ __device__ constexpr int att_keys(int qt) { return kVB * att_kb2(qt); }  // keys per LDS stage
#ifndef DG_ATT_NW
#define DG_ATT_NW 8
#endif
#ifndef DG_ATT_QT
#define DG_ATT_QT (8 / DG_ATT_NW)
#endif
constexpr int kNW = DG_ATT_NW;            // waves per workgroup (4 or 8)
constexpr int kQT = DG_ATT_QT;            // 16-query tiles per wave (share every K/V fragment read)
constexpr int kQTLarge = 2;               // the same for passes of more than 256 rows (prefill chunks)
#ifndef DG_ATT_LARGE_ROWS
#define DG_ATT_LARGE_ROWS 256
#endif
constexpr int kLargeRows = DG_ATT_LARGE_ROWS;  // passes of more rows take two query tiles per wave
// query tiles per wave for a pass of M rows: canvases keep one, so that their key range splits over
// more workgroups; long prefill chunks have work enough and share each staged K/V block among more
// queries
inline int attn_qt(int M) { return M > kLargeRows ? kQTLarge : kQT; }

// 2^x with the hardware instruction (about 1 ulp; 2^-inf = 0). Arguments here are <= 0.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int HD, int QT>
__global__ __launch_bounds__(64 * kNW) void attn_bf16_kernel(AttnArgs a) {
  constexpr int kWGRows = kNW * QT * 16;  // query rows per workgroup
  constexpr int HS = HD / 32;             // k-steps over head_dim
  constexpr int HT = HD / 16;             // O^T tiles over head_dim
  constexpr int ROWB = HD * 2;            // bytes per K row
  constexpr int CPR = ROWB / 16;          // 16-byte chunks per K row
  constexpr int kKB2 = att_kb2(QT);       // V blocks per stage
  constexpr int kKS = att_keys(QT);       // keys per stage
  constexpr int kStages = att_stages(QT); // LDS ring depth
  constexpr int KBYTES = kKS * ROWB;      // K bytes per stage
  constexpr int VBYTES = HD * kKS * 2;    // V^T bytes per stage (kKB2 blocks of [HD][32])
  constexpr int SBYTES = KBYTES + VBYTES;
  constexpr int CPW = SBYTES / (kNW * 1024);  // 1 KB wave copies per wave and stage
  constexpr int LPS = CPW;                     // loads per thread and stage
  static_assert(CPW >= 1 && CPW * kNW * 1024 == SBYTES && 1024 % ROWB == 0, "stage shape");
  __shared__ __align__(16) unsigned char smem[kStages * SBYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int rows_in_group = G * a.M;
  // block -> (query tile, KV head, split). The query tiles of one (KV head, split) read the same
  // K/V stream, so with the unit count a multiple of 8 they run on one XCD (block b on XCD b % 8).
  const int nunits = a.Hkv * a.splits;
  int qt, unit;
  if (nunits % 8 == 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    qt = j % a.qtiles;
    unit = (j / a.qtiles) * 8 + x;
  } else {
    qt = blockIdx.x % a.qtiles;
    unit = blockIdx.x / a.qtiles;
  }
  const int kvh = unit % a.Hkv;
  const int split = unit / a.Hkv;
  // the committed length may live on the device (a captured step serves every cache length): the
  // split count is then fixed by the host and each split's key range follows from the length
  int pos0 = a.pos0, key_chunk = a.key_chunk;
  if (a.pos_dev) {
    pos0 = *a.pos_dev;
    key_chunk = ((pos0 + a.M + a.splits - 1) / a.splits + kKS - 1) / kKS * kKS;
  }
  const int L = pos0 + a.M;
  const int g4 = lane >> 4, fr = lane & 15;

  int qr[QT], qhead[QT], qm[QT], qpos[QT];
  bool qvalid[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    qr[t] = qt * kWGRows + (wave * QT + t) * 16 + fr;
    qvalid[t] = qr[t] < rows_in_group;
    qhead[t] = kvh * G + (qvalid[t] ? qr[t] / a.M : 0);
    qm[t] = qvalid[t] ? qr[t] % a.M : 0;
    qpos[t] = pos0 + qm[t];
  }

  // key range of this split, clipped for causal attention to the workgroup's last position
  const int k_lo = split * key_chunk;
  int k_hi = min(L, k_lo + key_chunk);
  if (a.causal) {
    const int first_row = qt * kWGRows;
    const int last_row = min(rows_in_group - 1, first_row + kWGRows - 1);
    int maxpos = pos0 + a.M - 1;
    if (first_row / a.M == last_row / a.M) maxpos = pos0 + last_row % a.M;
    k_hi = min(k_hi, maxpos + 1);
  }
  const int nst = k_hi > k_lo ? (k_hi - k_lo + kKS - 1) / kKS : 0;

  // Q^T fragments (B operand): lane supplies query qr, head dims 8*g4 .. of each 32-step
  bf16x8_t qf[QT][HS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qm[t]) * a.ldq + qhead[t] * HD;
#pragma unroll
    for (int h = 0; h < HS; ++h) qf[t][h] = qvalid[t] ? Frag<bf16_t>::load(qb + h * 32 + g4 * 8) : Frag<bf16_t>::zero();
  }

  f32x4_t o[QT][HT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
#pragma unroll
    for (int j = 0; j < HT; ++j) o[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mrun[t] = -INFINITY;
    lrun[t] = 0.f;
  }

  // Copy sources. A stage is SBYTES / 1 KB wave copies, CPW per wave (copy c = wave * CPW + i); the
  // first KC are K: copy c covers rows c * RPC .. of the stage and lane l fills LDS position l % CPR
  // of row l / CPR with the row's chunk (l % CPR) ^ (row % CPR); rows past L re-read row L-1 (masked).
  // The rest are V^T (the stage's contiguous 32-position block): copy c covers hd rows
  // (c - KC) * 16 .., lane l fills position l % 4 of row l / 4 with chunk (l % 4) ^ ((row / 4) % 4).
  // With these swizzles the 16 rows a fragment read touches (16 lanes, 16 bytes each) fall on 16
  // distinct 16-byte bank groups: K row r's chunk q sits at position q ^ (r % CPR), and V^T rows of
  // 64 bytes put row r's chunk c at position c ^ ((r / 4) % 4).
  const bf16_t* kbase = static_cast<const bf16_t*>(a.kc) + kvh * a.head_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.vc) + kvh * a.head_stride;
  constexpr int RPC = 1024 / ROWB;
  constexpr int KC = KBYTES / 1024;
  int csrc[CPW];  // K: row within the stage * HD + chunk * 8; V: element offset in the block
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave * CPW + i;
    if (c < KC) {
      const int r = c * RPC + lane / CPR;
      csrc[i] = r * HD + ((lane % CPR) ^ (r & (CPR - 1))) * 8;
    } else {
      const int r = (c - KC) * 16 + lane / 4;  // row of the stage's [kKB2 * HD][32] V^T rows
      csrc[i] = r * kVB + ((lane % 4) ^ ((r >> 2) & 3)) * 8;
    }
  }
  auto issue = [&](int st, int slot) {
    const int key0 = k_lo + st * kKS;
    unsigned char* base = smem + slot * SBYTES;
    const bf16_t* vb = vbase + static_cast<int64_t>(key0 / kVB) * HD * kVB;
    const int kmax = (L - 1 - key0) * HD;  // element offset of row L-1 relative to key0
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = wave * CPW + i;
      if (c < KC) {
        const int off = csrc[i] <= kmax + (HD - 1) ? csrc[i] : kmax + (csrc[i] % HD);
        dma16(kbase + static_cast<int64_t>(key0) * HD + off, base + c * 1024);
      } else {
        // whole V blocks: a key range's last stage may copy up to att_keys - 32 positions past the
        // capacity, into the next head's blocks or the cache's tail (dg_kv_bytes); those keys are
        // masked, so the finite values there are weighted by zero
        dma16(vb + csrc[i], base + c * 1024);
      }
    }
  };

  // Q is in registers before the ring starts: the waits below then only count stage copies
  wait_vm_n<0>();
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u)
    if (u < nst) issue(u, u);
  for (int st = 0; st < nst; ++st) {
    wait_stages<LPS, kStages>(min(kStages - 2, nst - 1 - st));
    // stage st is in LDS for every wave, and every wave is done with stage st-1
    __builtin_amdgcn_s_barrier();
    if (st + kStages - 1 < nst) issue(st + kStages - 1, (st + kStages - 1) % kStages);
    const unsigned char* sk = smem + (st % kStages) * SBYTES;
    const unsigned char* sv = sk + KBYTES;
    const int key0 = k_lo + st * kKS;
    const bool need_mask = a.causal || key0 + kKS > k_hi;

    // K fragments of the stage (A operand of S^T = K Q^T), shared by the wave's query tiles
    constexpr int KT = kKS / 16;  // 16-key tiles per stage
    bf16x8_t kf[KT][HS];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int r = kt * 16 + fr;
#pragma unroll
      for (int h = 0; h < HS; ++h)
        kf[kt][h] = *reinterpret_cast<const bf16x8_t*>(sk + r * ROWB + (((h * 4 + g4) ^ (r & (CPR - 1))) << 4));
    }
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      f32x4_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HS; ++h) acc = Frag<bf16_t>::mma(kf[kt][h], qf[t][h], acc);
        s[kt] = acc;
      }
      // scale, mask (only stages that reach past k_hi, or causal ones), stage max over this lane's
      // keys and then the 4 lane groups
      float bmax = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + kt * 16 + g4 * 4 + i;
            const bool ok = key < k_hi && (!a.causal || key <= qpos[t]);
            s[kt][i] = ok ? s[kt][i] * a.scale_log2 : -INFINITY;
            bmax = fmaxf(bmax, s[kt][i]);
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[kt][i] *= a.scale_log2;
            bmax = fmaxf(bmax, s[kt][i]);
          }
      }
      bmax = xrow_max(bmax);
      const float mnew = fmaxf(mrun[t], bmax);
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // all masked so far: keep the base finite
      // rescale O and this lane's partial l only when some lane's running max grew (alpha = 1 otherwise)
      if (__any(mnew != mrun[t])) {
        const float alpha = fast_exp2(mrun[t] - mref);
        lrun[t] *= alpha;
#pragma unroll
        for (int j = 0; j < HT; ++j) o[t][j] *= alpha;
      }
      mrun[t] = mnew;
      // O^T += V^T P^T per V block: the P^T fragment of block b is key tiles 2b, 2b+1 (lane group g
      // holds keys 4g..4g+3 of each, the block's slot order); the V^T fragment of head dims
      // j*16 .. j*16+15 is row b * HD + j * 16 + lane % 16, slots 8*g4 .. 8*g4+7
#pragma unroll
      for (int b = 0; b < kKB2; ++b) {
        bf16x8_t pf;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(s[2 * b + u][i] - mref);
            lrun[t] += p;
            pf[u * 4 + i] = static_cast<__bf16>(p);
          }
#pragma unroll
        for (int j = 0; j < HT; ++j) {
          const int vr = b * HD + j * 16 + fr;
          const bf16x8_t vf =
              *reinterpret_cast<const bf16x8_t*>(sv + (vr * kVB + ((g4 ^ ((vr >> 2) & 3)) << 3)) * 2);
          o[t][j] = Frag<bf16_t>::mma(vf, pf, o[t][j]);
        }
      }
    }
  }

  // this lane's partial l covers its lane group's keys: sum the 4 groups
#pragma unroll
  for (int t = 0; t < QT; ++t) lrun[t] = xrow_sum(lrun[t]);

  // ---- results: lane holds O^T[hd = j*16 + 4*g4 + i][query qr]
  const int64_t R = static_cast<int64_t>(a.Hq) * a.M;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    if (!qvalid[t]) continue;
    if (a.splits == 1) {
      const float inv = lrun[t] > 0.f ? 1.0f / lrun[t] : 0.f;
      bf16_t* op = static_cast<bf16_t*>(a.o) + static_cast<int64_t>(qm[t]) * a.ldo + qhead[t] * HD;
#pragma unroll
      for (int j = 0; j < HT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) op[j * 16 + g4 * 4 + i] = f32_to_bf16(o[t][j][i] * inv);
      continue;
    }
    const int64_t row = static_cast<int64_t>(qhead[t]) * a.M + qm[t];
    float* po = a.part_o + (split * R + row) * HD;
#pragma unroll
    for (int j = 0; j < HT; ++j)
      *reinterpret_cast<float4*>(po + j * 16 + g4 * 4) = make_float4(o[t][j][0], o[t][j][1], o[t][j][2], o[t][j][3]);
    if (g4 == 0) {
      a.part_ml[(split * R + row) * 2] = mrun[t];
      a.part_ml[(split * R + row) * 2 + 1] = lrun[t];
    }
  }
}

// combine the key slices, one wave per query row, splits in a fixed order:
// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s. Every lane reads the (m, l) of all slices (the
// same addresses) so no cross-lane traffic is needed; lane l owns head dims 2l, 2l+1 (+128 ...).
// All slices' (m, l) loads are issued together, and the O rows in batches of 8 slices.
constexpr int kMergeMax = 32;  // attn_max_splits()
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int hd) {
  const int64_t R = static_cast<int64_t>(a.Hq) * a.M;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  const int S = a.splits;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  float2 e[kMergeMax];
#pragma unroll
  for (int s = 0; s < kMergeMax; ++s) e[s] = s < S ? ml[s * R + row] : make_float2(-INFINITY, 0.f);
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMergeMax; ++s) mx = fmaxf(mx, e[s].x);
  const int nc = hd / 128;  // float2 columns per lane beyond the first
  float l = 0.f;
  float2 acc[2] = {make_float2(0.f, 0.f), make_float2(0.f, 0.f)};
  constexpr int B = 8;
#pragma unroll
  for (int s0 = 0; s0 < kMergeMax; s0 += B) {
    if (s0 >= S) break;
    float2 v[B][2];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const float2* po = reinterpret_cast<const float2*>(a.part_o + ((s0 + q) * R + row) * hd);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        v[q][c] = (s0 + q < S && c <= nc && 2 * (lane + 64 * c) < hd) ? po[lane + 64 * c] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      if (s0 + q >= S) break;
      const float w = e[s0 + q].x == -INFINITY ? 0.f : exp2f(e[s0 + q].x - mx);
      l += w * e[s0 + q].y;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[c].x += w * v[q][c].x;
        acc[c].y += w * v[q][c].y;
      }
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const int head = static_cast<int>(row / a.M), m = static_cast<int>(row % a.M);
  T* out = static_cast<T*>(a.o) + static_cast<int64_t>(m) * a.ldo + head * hd;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int d = 2 * (lane + 64 * c);
    if (c <= nc && d < hd) {
      out[d] = from_f32<T>(acc[c].x * inv);
      out[d + 1] = from_f32<T>(acc[c].y * inv);
    }
  }
}

// fp32: one wave per (query row, head). Keys go 64 at a time, one per lane: the lane's score (its key
// row against the query, which the wave keeps in LDS), the chunk's maximum and sum by wave reductions
// into a running (max, sum) with the usual rescale. The chunk's probabilities go to LDS in the V cache's
// slot order, and each lane then accumulates head dims lane and lane + 64 over the chunk's two V blocks,
// reading the 32 contiguous slots of its dim's row in each block (kvlayout.h).
constexpr int kF32Waves = 4;
__global__ __launch_bounds__(64 * kF32Waves) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[kF32Waves][128];
  __shared__ __align__(16) float ps[kF32Waves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int idx = blockIdx.x * kF32Waves + wave;
  if (idx >= a.M * a.Hq) return;  // whole waves: no barrier below
  const int m = idx / a.Hq, j = idx % a.Hq;
  const int kvh = (j * a.Hkv) / a.Hq;
  const int hd = a.hd;
  const float* q = static_cast<const float*>(a.q) + static_cast<int64_t>(m) * a.ldq + j * hd;
  const float* kb = static_cast<const float*>(a.kc) + kvh * a.head_stride;
  const float* vb = static_cast<const float*>(a.vc) + kvh * a.head_stride;
  const int pos0 = a.pos_dev ? *a.pos_dev : a.pos0;
  const int L = a.causal ? pos0 + m + 1 : pos0 + a.M;
  float* qw = qs[wave];
  float* pw = ps[wave];
  for (int d = lane; d < hd; d += 64) qw[d] = q[d];
  // LDS written by this wave's own lanes is read by its other lanes after lgkmcnt(0); the compiler
  // barriers keep the accesses on their side of each wait
  auto lds_sync = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  lds_sync();
  float mrun = -INFINITY, lrun = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = 0; t0 < L; t0 += 64) {
    const int t = t0 + lane;
    float sc = -INFINITY;
    if (t < L) {
      const float4* kr = reinterpret_cast<const float4*>(kb + static_cast<int64_t>(t) * hd);
      float acc = 0.f;
      for (int d4 = 0; d4 < hd / 4; ++d4) {
        const float4 kv = kr[d4];
        acc += qw[4 * d4] * kv.x + qw[4 * d4 + 1] * kv.y + qw[4 * d4 + 2] * kv.z + qw[4 * d4 + 3] * kv.w;
      }
      sc = acc * a.scale_log2;
    }
    const float mnew = fmaxf(mrun, wave_max(sc));
    const float alpha = exp2f(mrun - mnew);  // 0 on the first chunk (mrun = -inf)
    const float p = t < L ? exp2f(sc - mnew) : 0.f;
    lrun = lrun * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    pw[(lane & 32) + v_slot(lane & 31)] = p;  // slot order inside each 32-position block
    lds_sync();
    const int nb = t0 + 32 < L ? 2 : 1;  // V blocks of the chunk holding keys (masked keys weigh 0)
    for (int b = 0; b < nb; ++b) {
      const float* blk = vb + (static_cast<int64_t>(t0 / 32 + b) * hd) * kVB;  // [hd][32] of the block
      const float4* pv = reinterpret_cast<const float4*>(pw + 32 * b);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int d = lane + 64 * c;
        if (d >= hd) break;
        const float4* row = reinterpret_cast<const float4*>(blk + d * kVB);
        float acc = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < 8; ++s4) {
          const float4 v = row[s4], pp = pv[s4];
          acc += v.x * pp.x + v.y * pp.y + v.z * pp.z + v.w * pp.w;
        }
        if (c == 0) o0 += acc; else o1 += acc;
      }
    }
    lds_sync();  // every lane has read pw before the next chunk writes it
    mrun = mnew;
  }
  float* o = static_cast<float*>(a.o) + static_cast<int64_t>(m) * a.ldo + j * hd;
  if (lane < hd) o[lane] = o0 / lrun;
  if (lane + 64 < hd) o[lane + 64] = o1 / lrun;
}

// ------------------------------------------------------------------- host
#ifndef DG_ATT_WGS
#define DG_ATT_WGS 256
#endif
constexpr int kAttnWGs = DG_ATT_WGS;  // target workgroups of a launch
int attn_max_splits() { return kMergeMax; }
constexpr int kVOverrun = (att_keys(1) > att_keys(kQTLarge) ? att_keys(1) : att_keys(kQTLarge)) - kVB;
static_assert(kVOverrun == 96, "the KV tail that dg.h documents (largest key stage - 32 positions)");
int attn_v_overrun() { return kVOverrun; }

// Upper bound of splits x M over the launches attention() makes for M query rows (the rows of its
// partial buffers).
int64_t attn_partial_rows(int M, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  const int wg_rows = kNW * attn_qt(M) * 16;
  const int qtiles = (G * M + wg_rows - 1) / wg_rows;
  const int splits = std::max(1, std::min(attn_max_splits(), (kAttnWGs + qtiles * Hkv - 1) / (qtiles * Hkv)));
  return static_cast<int64_t>(splits) * M;
}

// pos_dev (optional): the position of query row 0 is read on the device; the split count is then
// chosen for the largest position pos_max, so one launch configuration serves every length up to it.
int attention(const void* q, int64_t ldq, const void* kc, const void* vc, int64_t head_stride, int M, int Hq,
              int Hkv, int hd, int pos0, const int* pos_dev, int pos_max, int causal, float* part_o,
              float* part_ml, void* o, int64_t ldo, int dtype, hipStream_t s) {
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.kc = kc; a.vc = vc; a.head_stride = head_stride;
  a.M = M; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.pos0 = pos0; a.pos_dev = pos_dev; a.causal = causal;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(hd)));
  a.part_o = part_o; a.part_ml = part_ml; a.o = o; a.ldo = ldo;
  const int L = (pos_dev ? pos_max : pos0) + M;
  if (dtype == DG_F32) {
    if (hd > 128) return fail(DG_ERR_UNSUPPORTED, "fp32 attention needs head_dim <= 128");
    a.splits = 1;
    ProfScope ps("attention_f32", s);
    const int n = M * Hq;
    attn_f32_kernel<<<(n + kF32Waves - 1) / kF32Waves, 64 * kF32Waves, 0, s>>>(a);
    DG_LAUNCH_CHECK("attn_f32_kernel");
    return DG_OK;
  }
  if (hd != 64 && hd != 128) return fail(DG_ERR_UNSUPPORTED, "bf16 attention needs head_dim 64 or 128");
  const int G = Hq / Hkv;
  const int qt = attn_qt(M);
  const int kKS = att_keys(qt);
  const int wg_rows = kNW * qt * 16;
  const int qtiles = (G * M + wg_rows - 1) / wg_rows;
  // about 256 workgroups (one per CU; partial results cost HBM traffic per extra split), at least
  // four key stages per split
  int splits = std::max(1, std::min(attn_max_splits(), (kAttnWGs + qtiles * Hkv - 1) / (qtiles * Hkv)));
  splits = std::min(splits, std::max(1, (L + 4 * kKS - 1) / (4 * kKS)));
  a.key_chunk = ((L + splits - 1) / splits + kKS - 1) / kKS * kKS;
  // a host length drops the splits a rounded-up chunk leaves empty; a device length keeps them
  // (their key ranges depend on the length; an empty one contributes weight 0 to the merge)
  a.splits = pos_dev ? splits : (L + a.key_chunk - 1) / a.key_chunk;
  a.qtiles = qtiles;
  const dim3 grid(qtiles * Hkv * a.splits);
  {
    ProfScope ps("attention", s);
    if (qt == kQTLarge) {
      if (hd == 128) attn_bf16_kernel<128, kQTLarge><<<grid, 64 * kNW, 0, s>>>(a);
      else attn_bf16_kernel<64, kQTLarge><<<grid, 64 * kNW, 0, s>>>(a);
    } else {
      if (hd == 128) attn_bf16_kernel<128, kQT><<<grid, 64 * kNW, 0, s>>>(a);
      else attn_bf16_kernel<64, kQT><<<grid, 64 * kNW, 0, s>>>(a);
    }
  }
  DG_LAUNCH_CHECK("attn_bf16_kernel");
  if (a.splits == 1) return DG_OK;
  {
    ProfScope ps("attention_merge", s);
    const int64_t rows = static_cast<int64_t>(Hq) * M;
    attn_merge_kernel<bf16_t><<<static_cast<int>((rows + 3) / 4), 256, 0, s>>>(a, hd);
  }
  DG_LAUNCH_CHECK("attn_merge_kernel");
  return DG_OK;
}

}  // namespace dg
