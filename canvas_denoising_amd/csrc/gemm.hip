// Dense GEMM on the MFMA units: C = A * B^T (A activations [M x K], B weights
// stored [N x K]) with the epilogues the denoising step needs (store, residual
// add, GeLU, gated GeLU over paired gate/up rows, QKV split into the query
// buffer and the KV cache, MoE combine).
//
// Two tile kernels. bf16 (every GEMM of the benchmark model) runs
// gemm_dma_kernel: 64 x 64 tiles (128 x 128 for long prefill chunks) by 8
// waves, A and B rows of 128 bytes copied asynchronously from global memory
// straight into a 4-deep LDS ring (global_load_lds), chunks XOR-swizzled so
// fragment reads hit distinct banks, one counted wait and one barrier per
// k-tile. fp32 runs gemm_kernel: 4 waves in a 2 x 2 arrangement over the
// tile, rows padded by 16 bytes in LDS, a register prefetch of the next
// k-tile. In both, workgroups that share a B slice are mapped to the same XCD
// (dispatch is round-robin over the 8 XCDs) so the slice is fetched from HBM
// once and re-read from that XCD's L2, and split-K writes fp32 partials that
// a second kernel (or the caller's row kernel) reduces in a fixed order
// before the epilogue.
#include <algorithm>

#include "dg_common.h"
#include "gemm.h"
#include "mfma.h"
#include "dma.h"
#include "kvlayout.h"
#include "prof.h"

namespace dg {

template <typename T, int BM_, int BN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BK = 128 / static_cast<int>(sizeof(T));
  static constexpr int LDK = BK + 16 / static_cast<int>(sizeof(T));
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int VEC = 16 / static_cast<int>(sizeof(T));
  static constexpr int CHUNKS = BK / VEC;  // 8 sixteen-byte chunks per row
  static constexpr int A_LOADS = BM * CHUNKS / 256;
  static constexpr int B_LOADS = BN * CHUNKS / 256;
  static constexpr int KSTEPS = BK / 32;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");
  static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile");
};

template <typename T>
__device__ inline void epilogue(const GemmArgs& g, int row, int col, float v) {
  switch (g.epi) {
    case EPI_STORE:
      static_cast<T*>(g.out)[static_cast<int64_t>(row) * g.ldo + col] = from_f32<T>(v);
      break;
    case EPI_STORE_F32:
      static_cast<float*>(g.out)[static_cast<int64_t>(row) * g.ldo + col] = v;
      break;
    case EPI_ADD_F32:
      static_cast<float*>(g.out)[static_cast<int64_t>(row) * g.ldo + col] += v;
      break;
    case EPI_GELU:
      static_cast<T*>(g.out)[static_cast<int64_t>(row) * g.ldo + col] = from_f32<T>(gelu_erf(v));
      break;
    case EPI_QKV: {
      if (col < g.q_cols) {
        static_cast<T*>(g.out)[static_cast<int64_t>(row) * g.ldo + col] = from_f32<T>(v);
      } else {
        const int c = col - g.q_cols;
        const int per = g.n_kv * g.head_dim;
        const int which = c / per, rem = c - which * per;
        const int h = rem / g.head_dim, d = rem - h * g.head_dim;
        const int64_t pos = g.pos0 + row;
        if (which == 0)
          static_cast<T*>(g.kcache)[h * g.kv_head_stride + pos * g.head_dim + d] = from_f32<T>(v);
        else
          static_cast<T*>(g.vcache)[h * g.kv_head_stride + v_index(pos, d, g.head_dim)] = from_f32<T>(v);
      }
      break;
    }
    default:
      break;
  }
}

template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, int splits, int k_per_split) {
  if (g.epi == EPI_QKV && g.pos_dev) g.pos0 = *g.pos_dev;
  using C = GemmCfg<T, BM, BN>;
  using F = Frag<T>;
  __shared__ __align__(16) T sA[2][BM * C::LDK];
  __shared__ __align__(16) T sB[2][BN * C::LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool paired = g.epi == EPI_GEGLU;

  // ---- tile mapping: workgroups sharing an n-tile land on one XCD
  const int nm = (g.M + BM - 1) / BM;
  const int n_rows_b = g.N;  // rows of B visited (2F for paired)
  const int nn = (n_rows_b + BN - 1) / BN;
  const int b = blockIdx.x;
  const int nn8 = (nn / 8) * 8;
  int mt, nt;
  if (b < nm * nn8) {
    const int xcd = b & 7, j = b >> 3;
    nt = (j / nm) * 8 + xcd;
    mt = j % nm;
  } else {
    const int r = b - nm * nn8;
    nt = nn8 + r / nm;
    mt = r % nm;
  }
  const int m0 = mt * BM;
  const int z = blockIdx.y;
  const int k_begin = z * k_per_split;
  const int k_end = min(g.K, k_begin + k_per_split);
  const int nk = (k_end - k_begin) / C::BK;

  // B row of tile column t
  auto brow = [&](int t) -> int {
    if (!paired) return nt * BN + t;
    const int half = t / (BN / 2), c = t % (BN / 2);
    const int j0 = nt * (BN / 2) + half * (BN / 4);
    return c < BN / 4 ? j0 + c : g.pair_f + j0 + (c - BN / 4);
  };

  const T* A = static_cast<const T*>(g.A);
  const T* B = static_cast<const T*>(g.B);
  uint4 ra[C::A_LOADS], rb[C::B_LOADS];
  int arow[C::A_LOADS], achk[C::A_LOADS], brw[C::B_LOADS], bchk[C::B_LOADS];
  bool aok[C::A_LOADS], bok[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int q = tid + 256 * i;
    arow[i] = q / C::CHUNKS;
    achk[i] = q % C::CHUNKS;
    aok[i] = m0 + arow[i] < g.M;
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int q = tid + 256 * i;
    const int t = q / C::CHUNKS;
    bchk[i] = q % C::CHUNKS;
    brw[i] = t;
    bok[i] = paired ? true : (nt * BN + t < g.N);
  }
  int bsrc[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) bsrc[i] = bok[i] ? brow(brw[i]) : 0;

  auto gload = [&](int kt) {
    const int k0 = k_begin + kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      ra[i] = aok[i] ? *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(m0 + arow[i]) * g.lda + k0 +
                                                        achk[i] * C::VEC)
                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      rb[i] = bok[i] ? *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(bsrc[i]) * g.ldb + k0 +
                                                        bchk[i] * C::VEC)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      *reinterpret_cast<uint4*>(&sA[buf][arow[i] * C::LDK + achk[i] * C::VEC]) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      *reinterpret_cast<uint4*>(&sB[buf][brw[i] * C::LDK + bchk[i] * C::VEC]) = rb[i];
  };

  f32x4_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      typename F::type af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = F::load(&sA[cur][(wm * C::WM + i * 16 + fr) * C::LDK + ks * 32 + fk]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = F::load(&sB[cur][(wn * C::WN + j * 16 + fr) * C::LDK + ks * 32 + fk]);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = F::mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int rbase = m0 + wm * C::WM + (lane >> 4) * 4;
  if (splits > 1) {  // partial sums [z][row][B row] (gate j and up j of a paired GEMM at j, pair_f + j)
    float* part = g.part + static_cast<int64_t>(z) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int t = wn * C::WN + j * 16 + fr;
          const int col = paired ? brow(t) : nt * BN + t;
          if (row < g.M && col < g.N) part[static_cast<int64_t>(row) * g.N + col] = acc[i][j][r];
        }
    return;
  }
  if (paired) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN / 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int jj = nt * (BN / 2) + wn * (BN / 4) + j * 16 + fr;
          if (row < g.M) {
            const float v = gelu_erf(acc[i][j][r]) * acc[i][j + C::TN / 2][r];
            static_cast<T*>(g.out)[static_cast<int64_t>(row) * g.ldo + jj] = from_f32<T>(v);
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rbase + i * 16 + r;
        const int col = nt * BN + wn * C::WN + j * 16 + fr;
        if (row < g.M && col < g.N) epilogue<T>(g, row, col, acc[i][j][r]);
      }
}

// ---------------------------------------------------------------------------
// bf16 variant with a deep asynchronous pipeline. Loaded HBM latency is a few
// microseconds while one 64-deep k-tile of MFMA work takes a fraction of one,
// so a register double buffer leaves the kernel latency-bound. Here every
// wave issues global_load_lds_dwordx4 (gfx950: 16 bytes per lane straight
// into LDS, no registers) for k-tiles NS-1 ahead into a ring of NS LDS stages,
// waits with a counted s_waitcnt for the oldest stage only, and crosses one
// barrier per k-tile. A tile row is 128 bytes (8 chunks of 16); chunk q of row
// r is stored at position q ^ (r % 8) so the 16 rows a fragment read touches
// fall on different banks. Rows past M (or N) re-read the last valid row;
// their results are not stored.
template <int BM, int BN, int NS, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_dma_kernel(GemmArgs g, int splits, int k_per_split) {
  if (g.epi == EPI_QKV && g.pos_dev) g.pos0 = *g.pos_dev;
  // NW waves as (NW / 2) x 2 over the tile; every wave issues an equal share of the stage's copies
  constexpr int WM = BM / (NW / 2), WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int ROWB = 128;  // bytes per tile row: 64 bf16
  constexpr int SA = BM * ROWB, SB = BN * ROWB, SS = SA + SB;
  constexpr int ALPW = BM / (8 * NW), BLPW = BN / (8 * NW);  // load instructions per wave per stage (8 rows each)
  constexpr int LPS = ALPW + BLPW;
  static_assert(TM >= 1 && TN % 2 == 0 && ALPW >= 1 && BLPW >= 1, "tile");
  __shared__ __align__(16) unsigned char smem[NS * SS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool paired = g.epi == EPI_GEGLU;
  const int nm = (g.M + BM - 1) / BM;
  const int nn = (g.N + BN - 1) / BN;
  const int b = blockIdx.x;
  const int nn8 = (nn / 8) * 8;
  int mt, nt;
  if (b < nm * nn8) {
    const int xcd = b & 7, j = b >> 3;
    nt = (j / nm) * 8 + xcd;
    mt = j % nm;
  } else {
    const int r = b - nm * nn8;
    nt = nn8 + r / nm;
    mt = r % nm;
  }
  const int m0 = mt * BM;
  const int z = blockIdx.y;
  const int k_begin = z * k_per_split;
  const int k_end = min(g.K, k_begin + k_per_split);
  const int nk = (k_end - k_begin) / 64;

  auto brow = [&](int t) -> int {
    if (!paired) return min(nt * BN + t, g.N - 1);
    const int half = t / (BN / 2), c = t % (BN / 2);
    const int j0 = nt * (BN / 2) + half * (BN / 4);
    return c < BN / 4 ? j0 + c : g.pair_f + j0 + (c - BN / 4);
  };
  const bf16_t* A = static_cast<const bf16_t*>(g.A);
  const bf16_t* B = static_cast<const bf16_t*>(g.B);
  const bf16_t* asrc[ALPW];
  const bf16_t* bsrc[BLPW];
#pragma unroll
  for (int i = 0; i < ALPW; ++i) {
    const int r = (wave * ALPW + i) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ (r & 7);
    asrc[i] = A + static_cast<int64_t>(min(m0 + r, g.M - 1)) * g.lda + q * 8;
  }
#pragma unroll
  for (int i = 0; i < BLPW; ++i) {
    const int t = (wave * BLPW + i) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ (t & 7);
    bsrc[i] = B + static_cast<int64_t>(brow(t)) * g.ldb + q * 8;
  }
  auto issue = [&](int kt, int slot) {
    const int k0 = k_begin + kt * 64;
    unsigned char* base = smem + slot * SS;
#pragma unroll
    for (int i = 0; i < ALPW; ++i)
      dma16(asrc[i] + k0, base + (wave * ALPW + i) * 8 * ROWB);
#pragma unroll
    for (int i = 0; i < BLPW; ++i)
      dma16(bsrc[i] + k0, base + SA + (wave * BLPW + i) * 8 * ROWB);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_stages<LPS, NS>(min(NS - 2, nk - 1 - kt));  // leave the stages issued after this one in flight
    // Stage kt is complete for every wave, and every wave is done reading stage kt-1
    // (its fragments were consumed by MFMAs already issued). A bare s_barrier: the
    // fence of __syncthreads() would wait for all outstanding loads, draining the ring.
    __builtin_amdgcn_s_barrier();
    if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
    const unsigned char* sa = smem + (kt % NS) * SS;
    const unsigned char* sb = sa + SA;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[TM], bfr[TN];
      const int q = ks * 4 + g4;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + r * ROWB + ((q ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 16 + fr;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + r * ROWB + ((q ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Frag<bf16_t>::mma(af[i], bfr[j], acc[i][j]);
    }
  }

  // ---- epilogue (same mapping as gemm_kernel)
  const int rbase = m0 + wm * WM + (lane >> 4) * 4;
  if (splits > 1) {  // partial sums [z][row][B row], as gemm_kernel
    float* part = g.part + static_cast<int64_t>(z) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int t = wn * WN + j * 16 + fr;
          const int col = paired ? brow(t) : nt * BN + t;
          if (row < g.M && col < g.N) part[static_cast<int64_t>(row) * g.N + col] = acc[i][j][r];
        }
    return;
  }
  if (paired) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN / 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int jj = nt * (BN / 2) + wn * (BN / 4) + j * 16 + fr;
          if (row < g.M) {
            const float v = gelu_erf(acc[i][j][r]) * acc[i][j + TN / 2][r];
            static_cast<bf16_t*>(g.out)[static_cast<int64_t>(row) * g.ldo + jj] = f32_to_bf16(v);
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rbase + i * 16 + r;
        const int col = nt * BN + wn * WN + j * 16 + fr;
        if (row < g.M && col < g.N) epilogue<bf16_t>(g, row, col, acc[i][j][r]);
      }
}

constexpr int kSumBatch = 8;

// Sum the split-K partials in split order and apply the epilogue; a paired (gated GeLU) GEMM
// combines the gate sum at column j with the up sum at column pair_f + j.
template <typename T>
__global__ void splitk_reduce_kernel(GemmArgs g, int splits) {
  if (g.epi == EPI_QKV && g.pos_dev) g.pos0 = *g.pos_dev;
  const int64_t n = static_cast<int64_t>(g.M) * g.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  if (g.epi == EPI_GEGLU) {
    const int64_t nf = static_cast<int64_t>(g.M) * g.pair_f;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < nf; e += stride) {
      const int row = static_cast<int>(e / g.pair_f), j = static_cast<int>(e - static_cast<int64_t>(row) * g.pair_f);
      const int64_t gi = static_cast<int64_t>(row) * g.N + j;
      float gs = 0.f, us = 0.f;
      for (int z0 = 0; z0 < splits; z0 += kSumBatch) {  // loads issued together, summed in order
        float a[kSumBatch], b[kSumBatch];
#pragma unroll
        for (int q = 0; q < kSumBatch; ++q) {
          a[q] = z0 + q < splits ? g.part[(z0 + q) * n + gi] : 0.f;
          b[q] = z0 + q < splits ? g.part[(z0 + q) * n + gi + g.pair_f] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < kSumBatch; ++q) { gs += a[q]; us += b[q]; }
      }
      static_cast<T*>(g.out)[static_cast<int64_t>(row) * g.ldo + j] = from_f32<T>(gelu_erf(gs) * us);
    }
    return;
  }
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    float v = 0.f;
    for (int z0 = 0; z0 < splits; z0 += kSumBatch) {  // loads issued together, summed in order
      float a[kSumBatch];
#pragma unroll
      for (int q = 0; q < kSumBatch; ++q) a[q] = z0 + q < splits ? g.part[(z0 + q) * n + e] : 0.f;
#pragma unroll
      for (int q = 0; q < kSumBatch; ++q) v += a[q];
    }
    const int row = static_cast<int>(e / g.N), col = static_cast<int>(e - static_cast<int64_t>(row) * g.N);
    epilogue<T>(g, row, col, v);
  }
}

// ------------------------------------------------------------------- host
struct TileChoice { int bm, bn; };

// 128 x 128 tiles halve the operand traffic of 64 x 64 ones; they pay where the grid stays large
// (many column tiles) or K is long enough that split-K partials are small against the operands
// (the self-conditioning product over the vocabulary). Elsewhere, with a 256-row canvas, 64 x 64
// tiles give enough workgroups without splitting.
#ifndef DG_GEMM128_MIN_TILES
#define DG_GEMM128_MIN_TILES 256
#endif
static TileChoice pick_tile(int M, int N, int K) {
  const int64_t t128 = static_cast<int64_t>((M + 127) / 128) * ((N + 127) / 128);
  if (M > 64 && N >= 128 && (t128 >= DG_GEMM128_MIN_TILES || K >= 16384)) return {128, 128};
  return {64, 64};
}

#ifndef DG_GEMM_NS
#define DG_GEMM_NS 4
#endif
constexpr int kGemmStages64 = DG_GEMM_NS;  // LDS ring depth of the 64 x 64 tile
#ifndef DG_GEMM_NW
#define DG_GEMM_NW 8
#endif
constexpr int kGemmWaves64 = DG_GEMM_NW;   // waves of the 64 x 64 tile (4 or 8)
#ifndef DG_GEMM128_NS
#define DG_GEMM128_NS 2
#endif
#ifndef DG_GEMM128_NW
#define DG_GEMM128_NW 8
#endif
constexpr int kGemmStages128 = DG_GEMM128_NS;  // LDS ring depth of the 128 x 128 tile
constexpr int kGemmWaves128 = DG_GEMM128_NW;   // waves of the 128 x 128 tile (4 or 8)

#ifndef DG_GEMM_WGS
#define DG_GEMM_WGS 128
#endif
// Split-K grows the grid towards this many workgroups. At 128 the canvas's O projection and the
// shared expert's down projection (176 tiles) run unsplit: each takes a few microseconds longer,
// but the norm and the combine that read their output sum one plane instead of two, and the
// 30-layer loop measured 0.2-0.3 steps/s faster than with 256 (seven runs each, one box).
constexpr int64_t kGemmTargetWGs = DG_GEMM_WGS;

int gemm_pick_splits(int M, int N, int K, int dtype, int64_t part_capacity, bool allow_split) {
  if (!allow_split) return 1;
  const int bk = dtype == DG_BF16 ? 64 : 32;
  const TileChoice tc = pick_tile(M, N, K);
  const int64_t tiles = static_cast<int64_t>((M + tc.bm - 1) / tc.bm) * ((N + tc.bn - 1) / tc.bn);
  int s = 1;
  const int ktiles = K / bk;
  while (tiles * s < kGemmTargetWGs && s * 2 <= 32 && ktiles / (s * 2) >= 4 &&
         static_cast<int64_t>(s) * 2 * M * N <= part_capacity)
    s *= 2;
  return s;
}

template <typename T, int BM, int BN>
static int launch_tile(const GemmArgs& g, int splits, int kps, hipStream_t s) {
  const int nm = (g.M + BM - 1) / BM, nn = (g.N + BN - 1) / BN;
  dim3 grid(static_cast<unsigned>(nm * nn), static_cast<unsigned>(splits));
  gemm_kernel<T, BM, BN><<<grid, 256, 0, s>>>(g, splits, kps);
  DG_LAUNCH_CHECK("gemm_kernel");
  return DG_OK;
}

template <typename T>
static int gemm_t(const GemmArgs& g, int splits, hipStream_t s, const char* name) {
  const bool paired = g.epi == EPI_GEGLU;
  const int bk = 128 / static_cast<int>(sizeof(T));
  if (g.K % bk != 0) return fail(DG_ERR_UNSUPPORTED, std::string(name) + ": K must be a multiple of the k-tile");
  const TileChoice tc = pick_tile(g.M, g.N, g.K);
  if (paired && (g.pair_f % (tc.bn / 2) != 0 || g.N != 2 * g.pair_f))
    return fail(DG_ERR_UNSUPPORTED, std::string(name) + ": gated width must be a multiple of 32");
  const int ktiles = g.K / bk;
  const int kps = ((ktiles + splits - 1) / splits) * bk;
  splits = (g.K + kps - 1) / kps;
  if (splits > 1 && g.part == nullptr) return fail(DG_ERR_INVALID, "split-K needs scratch");
  int rc;
  {
    ProfScope ps(name, s);
    if constexpr (sizeof(T) == 2) {
      const int nm = (g.M + tc.bm - 1) / tc.bm, nn = (g.N + tc.bn - 1) / tc.bn;
      dim3 grid(static_cast<unsigned>(nm * nn), static_cast<unsigned>(splits));
      if (tc.bm == 128)
        gemm_dma_kernel<128, 128, kGemmStages128, kGemmWaves128><<<grid, 64 * kGemmWaves128, 0, s>>>(g, splits, kps);
      else gemm_dma_kernel<64, 64, kGemmStages64, kGemmWaves64><<<grid, 64 * kGemmWaves64, 0, s>>>(g, splits, kps);
      rc = DG_OK;
    } else {
      if (tc.bm == 128) rc = launch_tile<T, 128, 128>(g, splits, kps, s);
      else rc = launch_tile<T, 64, 64>(g, splits, kps, s);
    }
  }
  DG_LAUNCH_CHECK("gemm_dma_kernel");
  if (rc != DG_OK) return rc;
  if (g.splits_out) *g.splits_out = splits;
  if (splits > 1 && !g.defer_reduce) {
    ProfScope ps("splitk_reduce", s);
    const int64_t n = static_cast<int64_t>(g.M) * g.N;
    const int grid = static_cast<int>(std::min<int64_t>((n + 255) / 256, 4096));
    splitk_reduce_kernel<T><<<grid, 256, 0, s>>>(g, splits);
    DG_LAUNCH_CHECK("splitk_reduce_kernel");
  }
  return DG_OK;
}

int gemm(const GemmArgs& g, int dtype, int splits, hipStream_t s, const char* name) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return DG_OK;
  return dtype == DG_BF16 ? gemm_t<bf16_t>(g, splits, s, name) : gemm_t<float>(g, splits, s, name);
}

}  // namespace dg
