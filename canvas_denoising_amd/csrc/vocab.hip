// LM head of the denoiser: logits[M x V] = h[M x D] E^T over the tied
// embedding ([P3] "Encoder-denoiser design": logits are produced at every
// canvas position; [P4] "Gemma-based MoE backbone", table: vocabulary of
// 262144 tokens).
//
// With a canvas of M <= 256 rows the weight matrix E (V x D, 1.5 GB at the
// benchmark shape) is the stream: every E row is read exactly once, straight
// from HBM into MFMA B fragments. E is stored fragment-tiled with groups of
// 32 rows (tiles.h), so a wave's stream is one contiguous run. The rows of
// h are shared by every wave, so they are staged per 128-byte k-tile into an
// LDS ring (asynchronous global->LDS copies, XOR-swizzled rows, dma.h) and
// each wave multiplies all M rows against its 32 columns: 16 x 2 fragment
// accumulators, every A fragment read from LDS feeding two MFMAs.
//
// The self-conditioning product u = P E (P the tempered distribution of the
// previous step, [M x V]; [P3] "Inference mechanism") has the same shape with
// the roles of the dimensions exchanged: P is the staged operand, the
// transposed embedding E^T (D x V, tiled the same way) the stream, and K = V.
// P is never stored: the kernel loads the logits, forms
// p = 2^(l c - b_r) with c = log2(e) / T and b_r = m_r c + ln(Z_r) log2(e)
// from the sampler's row statistics (m_r, ln Z_r), and writes the bf16 / fp32
// probabilities into the LDS ring where the LM head's copies would land. Its
// D / 256 column blocks alone would occupy only a few compute units, so the
// vocabulary is also split into k shares; the fp32 partials of the shares are
// summed in order by a second kernel. The column blocks of one k share run on
// one XCD (the dispatcher sends block b to XCD b % 8), so the logits rows
// they all read are fetched into that XCD's L2 once.
//
// One loop iteration per k-tile: wait until the copies of the k-tile have
// landed (each wave issues exactly 8 loads per k-tile, 4 copies into LDS and 4
// register loads of E, so a fixed vmcnt leaves the younger k-tiles in flight),
// one barrier, issue the k-tile NS-1 ahead (k-tiles past the end re-read the
// last one and are never used), multiply. Self-conditioning copies the raw
// logits the same way, one k-tile further ahead (a ring of 4): at iteration
// kt, while the MFMAs of k-tile kt run, every lane turns the pieces its own
// copies of k-tile kt+1 wrote into probabilities in place (its own wave's
// vmcnt says they have landed, and no other lane touches them); the next
// iteration's barrier publishes them.
#include <algorithm>

#include "dg_common.h"
#include "dma.h"
#include "entrec.h"
#include "mfma.h"
#include "prof.h"
#include "tiles.h"

namespace dg {

constexpr int kVW = 8;         // waves per workgroup
constexpr int kVRows = 256;    // rows of h staged per k-tile (M <= 256)
constexpr int kVNS = 3;        // ring depth (k-tiles) of the LM head
constexpr int kVNSsc = 4;      // ring depth of the self-conditioning product
constexpr int kVRowB = 128;    // bytes of one h row per k-tile
constexpr int kMaxSplitSum = 32;  // most k shares of the split form

template <typename T>
__device__ inline typename Frag<T>::type lds_frag(const unsigned char* stage, int r, int ks, int g4);

template <>
__device__ inline bf16x8_t lds_frag<bf16_t>(const unsigned char* stage, int r, int ks, int g4) {
  const int q = ks * 4 + g4;
  return *reinterpret_cast<const bf16x8_t*>(stage + r * kVRowB + ((q ^ (r & 7)) << 4));
}

template <>
__device__ inline f32x8_t lds_frag<float>(const unsigned char* stage, int r, int ks, int g4) {
  (void)ks;
  const int q = 2 * g4;
  const float4 lo = *reinterpret_cast<const float4*>(stage + r * kVRowB + ((q ^ (r & 7)) << 4));
  const float4 hi = *reinterpret_cast<const float4*>(stage + r * kVRowB + (((q + 1) ^ (r & 7)) << 4));
  f32x8_t f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

enum VocabMode : int { kLmHead = 0, kSelfCond = 1, kLmHeadStats = 2 };

// Grid: ceil(V / (32 kVW)) workgroups of kVW waves; wave w of block b owns vocabulary group
// b * kVW + w (E rows 32 g .. 32 g + 31).
// kSelfCond: the split-k form. Block b: slot q = (b % 8) J + b / 8 (J = grid / 8) names k share q / nblk
// and column block q % nblk; its k-tiles are [KT s / S, KT (s + 1) / S); `h` holds the logits [M x K]
// (row stride ldh), stats [M x 2] their rows' (max, ln Z) and *temp the temperature; it stores fp32
// partials part[s][row][col] (row stride ldo) instead of T outputs.
template <typename T, int MODE>
__global__ __launch_bounds__(64 * kVW) void vocab_gemm_kernel(const T* __restrict__ h, int64_t ldh,
                                                             const T* __restrict__ E, int M, int V, int D,
                                                             T* __restrict__ logits, int64_t ldo,
                                                             float* __restrict__ part, int S, int nblk,
                                                             const float* __restrict__ stats,
                                                             const float* __restrict__ temp) {
  constexpr bool SC = MODE == kSelfCond;
  constexpr int NS = kVNS;                                  // register ring of E fragments (k-tiles)
  constexpr int NA = SC ? kVNSsc : kVNS;                    // LDS ring of A stages
  constexpr int KE = kVRowB / static_cast<int>(sizeof(T));  // k elements per k-tile
  constexpr int KS = KE / 32;                               // MFMA k-steps per k-tile
  constexpr int SBYTES = kVRows * kVRowB;                   // 32 KB per stage
  constexpr int CPW = SBYTES / (kVW * 1024);                // 1 KB copies per wave per k-tile (4)
  constexpr int BF = 2 * KS;                                // B fragments per k-tile
  using FT = typename Frag<T>::type;
  static_assert(CPW == 4, "8 loads per k-tile: 4 copies + 4 register loads");
  static_assert((sizeof(T) == 2 && BF == 4) || (sizeof(T) == 4 && BF == 2), "B loads per k-tile");
  __shared__ __align__(16) unsigned char smem[NA * SBYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  int blk = blockIdx.x, ks = 0, kbeg = 0, KT = D / KE;
  if constexpr (SC) {
    const int J = gridDim.x / 8;
    const int q = (blockIdx.x & 7) * J + (blockIdx.x >> 3);
    if (q >= nblk * S) return;  // padding block of the XCD-aware grid: no barrier reached
    ks = q / nblk;
    blk = q - ks * nblk;
    const int kt_all = KT;
    kbeg = static_cast<int>(static_cast<int64_t>(kt_all) * ks / S);
    KT = static_cast<int>(static_cast<int64_t>(kt_all) * (ks + 1) / S) - kbeg;
  }
  const int grp = blk * kVW + wave;
  const bool active = grp * 32 < V;  // idle waves run the loop on group 0 (uniform barriers), store nothing

  // A copies: copy c = wave * CPW + i covers rows 8c .. 8c+7 of the stage; lane l fills position l % 8
  // of row 8c + l / 8 with the row's chunk (l % 8) ^ (row % 8). Rows past M re-read row M-1. (Element
  // offsets from h: M <= 256 rows of at most 2^23 elements fit in 32 bits.)
  int aoff[CPW];
  float arow_b[CPW];  // self-conditioning: b_r = m_r c + ln(Z_r) log2(e) of the copy's row
  float pc = 0.f;     // c = log2(e) / T
  if constexpr (SC) pc = kLog2e / *temp;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (wave * CPW + i) * 8 + lane / 8;
    const int rc = min(r, M - 1);
    aoff[i] = rc * static_cast<int>(ldh) + ((lane % 8) ^ (r & 7)) * (16 / static_cast<int>(sizeof(T)));
    if constexpr (SC) arow_b[i] = fmaf(stats[2 * rc], pc, stats[2 * rc + 1] * kLog2e);
    else arow_b[i] = 0.f;
  }
  // B: this lane's fragment of k-tile 0 of the wave's group (inactive waves re-read group 0)
  const T* bsrc = E + static_cast<int64_t>(active ? grp : 0) * (D / 32) * 2 * kTileElems + lane * 8;

  FT breg[NS][BF];
  auto issue_a = [&](int kt, int aslot) {
    const int k = kbeg + min(kt, KT - 1);
    unsigned char* base = smem + aslot * SBYTES;
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(h + aoff[i] + k * KE, base + (wave * CPW + i) * 1024);
  };
  auto issue_b = [&](int kt, int slot) {
    const int k = kbeg + min(kt, KT - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int n = 0; n < 2; ++n)
        breg[slot][s * 2 + n] = Frag<T>::load(bsrc + (static_cast<int64_t>(k * KS + s) * 2 + n) * kTileElems);
  };
  // self-conditioning: the logits this lane's copies wrote into slot `slot` become probabilities in
  // place. In 16 units (piece i, word j: two logits) so that compute() can interleave them with its MFMAs.
  auto prob_word = [&](uint32_t w, float b) -> uint32_t {
    if constexpr (sizeof(T) == 2) {
      return pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(bf16lo(w), pc, -b)),
                         __builtin_amdgcn_exp2f(fmaf(bf16hi(w), pc, -b)));
    } else {
      return __float_as_uint(__builtin_amdgcn_exp2f(fmaf(__uint_as_float(w), pc, -b)));
    }
  };
  auto probs_in_place = [&](int slot) {
    unsigned char* base = smem + slot * SBYTES + lane * 16;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      uint4* pp = reinterpret_cast<uint4*>(base + (wave * CPW + i) * 1024);
      const uint4 v = *pp;
      *pp = make_uint4(prob_word(v.x, arow_b[i]), prob_word(v.y, arow_b[i]), prob_word(v.z, arow_b[i]),
                       prob_word(v.w, arow_b[i]));
    }
  };

  f32x4_t acc[16][2];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m][0] = acc[m][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // all 16 row tiles are multiplied (rows past M repeat row M-1 and are not stored): no branches
  // in the loop body, so the compiler's own waits for the E registers stay counted, not drained
  auto compute = [&](int aslot, int slot) {
    const unsigned char* st = smem + aslot * SBYTES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const FT af = lds_frag<T>(st, m * 16 + fr, s, g4);
        acc[m][0] = Frag<T>::mma(af, breg[slot][s * 2 + 0], acc[m][0]);
        acc[m][1] = Frag<T>::mma(af, breg[slot][s * 2 + 1], acc[m][1]);
      }
    }
  };
  // self-conditioning: compute(aslot, slot) with the conversion of stage cslot spread between the
  // MFMAs (a unit of two logits after every 32 / 16 = 2 fragment pairs), so that the exponentials run
  // while the matrix cores work instead of after them
  auto compute_sc = [&](int aslot, int slot, int cslot) {
    const unsigned char* st = smem + aslot * SBYTES;
    uint4* cp = reinterpret_cast<uint4*>(smem + cslot * SBYTES + lane * 16 + wave * CPW * 1024);
    uint4 raw = cp[0], next = raw;  // piece i, and piece i+1 read ahead (1 KB apart: 64 uint4)
    uint32_t out[4];
    constexpr int kSteps = KS * 16;             // fragment pairs of one k-tile
    constexpr int kEvery = kSteps / (CPW * 4);  // pairs between conversion units
    static_assert(kEvery >= 1 && kSteps % (CPW * 4) == 0, "conversion units per k-tile");
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const FT af = lds_frag<T>(st, m * 16 + fr, s, g4);
        acc[m][0] = Frag<T>::mma(af, breg[slot][s * 2 + 0], acc[m][0]);
        acc[m][1] = Frag<T>::mma(af, breg[slot][s * 2 + 1], acc[m][1]);
        const int t = s * 16 + m;
        if (t % kEvery == kEvery - 1) {
          const int q = t / kEvery, i = q / 4, j = q % 4;
          if (j == 0 && i + 1 < CPW) next = cp[(i + 1) * 64];
          const uint32_t w = j == 0 ? raw.x : j == 1 ? raw.y : j == 2 ? raw.z : raw.w;
          out[j] = prob_word(w, arow_b[i]);
          if (j == 3) {
            cp[i * 64] = make_uint4(out[0], out[1], out[2], out[3]);
            raw = next;
          }
        }
      }
    }
  };
  // u = kt % NS selects the E registers (compile-time); the LDS stage of k-tile kt is kt % NA.
  // LM head: the copies of k-tile kt+2 go out with its E loads (8 loads a k-tile).
  // Self-conditioning: iteration kt issues the copies of k-tile kt+3 and the E loads of kt+2, so
  // at its start the oldest group in flight is (copies of kt+1, E of kt).
  auto step = [&](int kt, int u) {
    if constexpr (SC) {
      wait_vm_n<8>();  // the copies of k-tile kt+1 and the E fragments of kt have landed
      // this wave's conversion of k-tile kt (the previous iteration) has completed (lgkmcnt(0)); the
      // compiler barriers keep every LDS access on its side of the workgroup barrier
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();  // k-tile kt is probabilities for all waves; all are done with kt-1
      asm volatile("" ::: "memory");
      issue_a(kt + 3, (kt + 3) % NA);
      issue_b(kt + 2, (u + 2) % NS);
      compute_sc(kt % NA, u, (kt + 1) % NA);  // k-tile kt, and k-tile kt+1 into probabilities
    } else {
      wait_vm_n<(NS - 2) * 8>();
      __builtin_amdgcn_s_barrier();  // k-tile kt is in LDS for all waves; all are done with kt-1
      issue_a(kt + NS - 1, (u + NS - 1) % NS);
      issue_b(kt + NS - 1, (u + NS - 1) % NS);
      compute(u, u);
    }
  };

  static_assert(!SC || (NS == 3 && NA == 4), "self-conditioning rings: E 2 k-tiles ahead, copies 3 ahead");
  if constexpr (SC) {
    issue_a(0, 0);
    issue_a(1, 1);
    issue_b(0, 0);
    issue_a(2, 2);
    issue_b(1, 1);
    wait_vm_n<16>();  // the copies of k-tile 0 have landed
    asm volatile("" ::: "memory");
    probs_in_place(0);  // published by the first iteration's barrier
  } else {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      issue_a(u, u);
      issue_b(u, u);
    }
  }
  int k0 = 0;
  for (; k0 + NS <= KT; k0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(k0 + u, u);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (k0 + u < KT) step(k0 + u, u);
  wait_vm_n<0>();  // the trailing (never used) copies have landed before the workgroup retires
  if constexpr (MODE == kLmHeadStats) {
    // The block's logits leave through LDS in two halves of 128 rows (each wave its 128 x 32 tile,
    // 8 KB, in the ring's first 64 KB), so that every lane stores 64 contiguous bytes of a row and
    // folds that row's 32 values (as stored, bf16) into a split-row record at temperature *temp;
    // the 8 waves' records of a row then merge in wave order into the block's record,
    // part[row * gridDim.x + blockIdx.x] (Rec layout).
    const float c = kLog2e / *temp;
    // lane indices re-derived here (opaque to the compiler), so that no epilogue address is computed
    // ahead of the k-loop and held through it
    int xl = lane, xt = tid;
    asm volatile("" : "+v"(xl), "+v"(xt));
    const int lane_e = xl, fr_e = xl & 15, g4_e = xl >> 4, tid_e = xt;
    __syncthreads();  // every wave is done with the ring
    unsigned char* tile = smem + wave * 8192;
    Rec* wrec = reinterpret_cast<Rec*>(smem + kVW * 8192);  // [256 rows][kVW waves]
    static_assert(kVW * 8192 + kVRows * kVW * sizeof(Rec) <= NA * SBYTES, "epilogue LDS");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int mm = 0; mm < 8; ++mm)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            reinterpret_cast<bf16_t*>(tile)[(mm * 16 + g4_e * 4 + i) * 32 + n * 16 + fr_e] =
                f32_to_bf16(acc[half * 8 + mm][n][i]);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rl = 2 * lane_e + q, row = half * 128 + rl;
        const uint4* src = reinterpret_cast<const uint4*>(tile + rl * 64);
        uint4 w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = src[k];
        if (active && row < M) {
          uint4* dst = reinterpret_cast<uint4*>(logits + static_cast<int64_t>(row) * ldo + grp * 32);
#pragma unroll
          for (int k = 0; k < 4; ++k) dst[k] = w[k];
        }
        float v[32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t x[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            v[k * 8 + 2 * h] = bf16lo(x[h]);
            v[k * 8 + 2 * h + 1] = bf16hi(x[h]);
          }
        }
        float m = v[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) m = fmaxf(m, v[j]);
        int first = 31;
#pragma unroll
        for (int j = 30; j >= 0; --j)
          if (v[j] == m) first = j;
        const float off = -m * c;
        float z = 0.f, a = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float u = fmaf(v[j], c, off);
          const float e = __builtin_amdgcn_exp2f(u);
          z += e;
          a = fmaf(u, e, a);
        }
        wrec[row * kVW + wave] = active ? Rec{m, z, a, grp * 32 + first} : Rec{-INFINITY, 0.f, 0.f, 0x7FFFFFFF};
      }
      __syncthreads();  // the tiles are rewritten by the next half; the records are complete
    }
    if (tid_e < kVRows && tid_e < M) {
      Rec r = wrec[tid_e * kVW];
#pragma unroll
      for (int w2 = 1; w2 < kVW; ++w2) rec_merge(r, wrec[tid_e * kVW + w2], c);
      reinterpret_cast<Rec*>(part)[static_cast<int64_t>(tid_e) * gridDim.x + blockIdx.x] = r;
    }
    return;
  }
  if (!active) return;
  // lane holds C[row = m*16 + 4*g4 + i][col = 32 grp + n*16 + fr]
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m * 16 + g4 * 4 + i;
      if (row < M) {
        if constexpr (SC) {
          float* o = part + (static_cast<int64_t>(ks) * M + row) * ldo + grp * 32 + fr;
          o[0] = acc[m][0][i];
          o[16] = acc[m][1][i];
        } else {
          T* o = logits + static_cast<int64_t>(row) * ldo + grp * 32 + fr;
          o[0] = from_f32<T>(acc[m][0][i]);
          o[16] = from_f32<T>(acc[m][1][i]);
        }
      }
    }
}

// out[row][col] = sum over s = 0 .. S-1, in order, of part[s][row][col] (N % 4 == 0); 4 columns per thread
template <typename T>
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int S, int M, int N,
                                                        T* __restrict__ out) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n4 = static_cast<int64_t>(M) * N / 4;
  if (i4 >= n4) return;
  const float4* p = reinterpret_cast<const float4*>(part);
  float4 v[kMaxSplitSum];
#pragma unroll
  for (int q = 0; q < kMaxSplitSum; ++q) v[q] = q < S ? p[q * n4 + i4] : float4{0.f, 0.f, 0.f, 0.f};
  float4 a = v[0];
#pragma unroll
  for (int q = 1; q < kMaxSplitSum; ++q) {
    a.x += v[q].x; a.y += v[q].y; a.z += v[q].z; a.w += v[q].w;
  }
  T* o = out + i4 * 4;
  o[0] = from_f32<T>(a.x); o[1] = from_f32<T>(a.y); o[2] = from_f32<T>(a.z); o[3] = from_f32<T>(a.w);
}

int vocab_gemm(const void* h, int64_t ldh, const void* E, int M, int V, int D, void* logits, int64_t ldo, int dtype,
               hipStream_t s) {
  if (M < 1 || M > kVRows) return fail(DG_ERR_UNSUPPORTED, "LM head: rows must be in [1, 256]");
  const int ke = dtype == DG_BF16 ? 64 : 32;
  if (D % ke != 0 || V % 32 != 0) return fail(DG_ERR_UNSUPPORTED, "LM head: d_model / vocab do not tile");
  if (static_cast<int64_t>(M) * ldh + D > INT32_MAX) return fail(DG_ERR_UNSUPPORTED, "LM head: rows too long");
  const int grid = (V / 32 + kVW - 1) / kVW;
  ProfScope ps("lm_head", s);
  if (dtype == DG_BF16)
    vocab_gemm_kernel<bf16_t, kLmHead><<<grid, 64 * kVW, 0, s>>>(static_cast<const bf16_t*>(h), ldh,
                                                                  static_cast<const bf16_t*>(E), M, V, D,
                                                                  static_cast<bf16_t*>(logits), ldo, nullptr, 1, 0,
                                                                  nullptr, nullptr);
  else
    vocab_gemm_kernel<float, kLmHead><<<grid, 64 * kVW, 0, s>>>(static_cast<const float*>(h), ldh,
                                                                 static_cast<const float*>(E), M, V, D,
                                                                 static_cast<float*>(logits), ldo, nullptr, 1, 0,
                                                                 nullptr, nullptr);
  DG_LAUNCH_CHECK("vocab_gemm_kernel");
  return DG_OK;
}

int vocab_gemm_stats(const void* h, int64_t ldh, const void* E, int M, int V, int D, void* logits, int64_t ldo,
                     const float* temp, void* recs, int dtype, hipStream_t s) {
  if (dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "LM head with sampler records: bf16 only");
  if (M < 1 || M > kVRows) return fail(DG_ERR_UNSUPPORTED, "LM head: rows must be in [1, 256]");
  if (D % 64 != 0 || V % 32 != 0) return fail(DG_ERR_UNSUPPORTED, "LM head: d_model / vocab do not tile");
  if (ldo % 8 != 0 || reinterpret_cast<uintptr_t>(logits) % 16 != 0)
    return fail(DG_ERR_UNSUPPORTED, "LM head with records: logits rows must be 16-byte aligned");
  if (static_cast<int64_t>(M) * ldh + D > INT32_MAX) return fail(DG_ERR_UNSUPPORTED, "LM head: rows too long");
  const int grid = (V / 32 + kVW - 1) / kVW;
  ProfScope ps("lm_head", s);
  vocab_gemm_kernel<bf16_t, kLmHeadStats><<<grid, 64 * kVW, 0, s>>>(
      static_cast<const bf16_t*>(h), ldh, static_cast<const bf16_t*>(E), M, V, D, static_cast<bf16_t*>(logits), ldo,
      static_cast<float*>(recs), 1, 0, nullptr, temp);
  DG_LAUNCH_CHECK("vocab_gemm_kernel");
  return DG_OK;
}

int vocab_blocks(int V) { return (V / 32 + kVW - 1) / kVW; }

int sc_embed_splits(int N, int64_t K, int dtype) {
  const int ke = dtype == DG_BF16 ? 64 : 32;
  const int nblk = (N / 32 + kVW - 1) / kVW;
  const int64_t kt = K / ke;
  int S = std::max(1, std::min(kMaxSplitSum, 256 / nblk));
  while (S > 1 && kt / S < 8) --S;  // at least 8 k-tiles per share
  return S;
}

int sc_embed(const void* logits, int64_t ldl, const float* stats, const float* temp, const void* Et, int M, int N,
             int64_t K, float* part, void* u, int dtype, hipStream_t s) {
  if (M < 1 || M > kVRows) return fail(DG_ERR_UNSUPPORTED, "self-conditioning: rows must be in [1, 256]");
  const int ke = dtype == DG_BF16 ? 64 : 32;
  if (K % ke != 0 || N % 32 != 0 || K > (int64_t{1} << 30))
    return fail(DG_ERR_UNSUPPORTED, "self-conditioning: vocab / d_model do not tile");
  if (static_cast<int64_t>(M) * ldl + K > INT32_MAX)
    return fail(DG_ERR_UNSUPPORTED, "self-conditioning: canvas x vocab too large");
  const int nblk = (N / 32 + kVW - 1) / kVW;
  const int S = sc_embed_splits(N, K, dtype);
  const int grid = 8 * ((nblk * S + 7) / 8);
  {
    ProfScope ps("sc_embed", s);
    if (dtype == DG_BF16)
      vocab_gemm_kernel<bf16_t, kSelfCond><<<grid, 64 * kVW, 0, s>>>(
          static_cast<const bf16_t*>(logits), ldl, static_cast<const bf16_t*>(Et), M, N, static_cast<int>(K),
          nullptr, N, part, S, nblk, stats, temp);
    else
      vocab_gemm_kernel<float, kSelfCond><<<grid, 64 * kVW, 0, s>>>(
          static_cast<const float*>(logits), ldl, static_cast<const float*>(Et), M, N, static_cast<int>(K),
          nullptr, N, part, S, nblk, stats, temp);
  }
  DG_LAUNCH_CHECK("vocab_gemm_kernel");
  {
    ProfScope ps("sc_sum", s);
    const int64_t n4 = static_cast<int64_t>(M) * N / 4;
    const unsigned g = static_cast<unsigned>((n4 + 255) / 256);
    if (dtype == DG_BF16) split_sum_kernel<bf16_t><<<g, 256, 0, s>>>(part, S, M, N, static_cast<bf16_t*>(u));
    else split_sum_kernel<float><<<g, 256, 0, s>>>(part, S, M, N, static_cast<float*>(u));
  }
  DG_LAUNCH_CHECK("split_sum_kernel");
  return DG_OK;
}

}  // namespace dg
