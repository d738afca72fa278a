// Dense MFMA GEMM of libdg: C[M x N] = A[M x K] * B[N x K]^T with fused epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum GemmEpi : int {
  EPI_STORE = 0,      // out[T][row*ldo + col] = v
  EPI_STORE_F32 = 1,  // out[f32] = v
  EPI_ADD_F32 = 2,    // out[f32] += v            (residual add)
  EPI_GELU = 3,       // out[T] = GeLU(v)
  EPI_GEGLU = 4,      // paired B rows: out[T][row*ldo + j] = GeLU(gate_j) * up_j
  EPI_QKV = 5,        // col < q_cols -> q out[T]; else K / V cache rows pos0 + row
};

struct GemmArgs {
  const void* A = nullptr;  // [M x K] row-major, lda elements
  int64_t lda = 0;
  const void* B = nullptr;  // [N x K] row-major (weights [out, in]), ldb elements
  int64_t ldb = 0;
  int M = 0, N = 0, K = 0;
  int epi = EPI_STORE;
  void* out = nullptr;
  int64_t ldo = 0;
  // EPI_GEGLU: N counts gate+up rows (2F); up rows start at row pair_f of B
  int pair_f = 0;
  // EPI_QKV
  int q_cols = 0, head_dim = 0, n_kv = 0, pos0 = 0;
  const int* pos_dev = nullptr;  // when set, the cache position of row 0 is *pos_dev (read on the device)
  int64_t kv_head_stride = 0;  // elements between KV heads (capacity * head_dim)
  void* kcache = nullptr;
  void* vcache = nullptr;
  // split-K scratch: splits * M * N floats
  float* part = nullptr;
  // leave split-K partials unreduced (the caller folds them into a row kernel); gemm() then
  // reports the split count through *splits_out
  bool defer_reduce = false;
  int* splits_out = nullptr;
};

// dtype: DG_BF16 / DG_F32. splits > 1 requires g.part and an epilogue other than GEGLU.
int gemm(const GemmArgs& g, int dtype, int splits, hipStream_t s, const char* name);
// splits the launcher would choose for this shape given `part_capacity` floats of scratch
int gemm_pick_splits(int M, int N, int K, int dtype, int64_t part_capacity, bool allow_split);

}  // namespace dg
