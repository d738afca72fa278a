// KV cache layout of libdg, per layer and KV head, for `cap` positions
// (cap a multiple of 32):
//   K: [cap][head_dim], row-major.
//   V: [cap / 32][head_dim][32]: V transposed in blocks of 32 positions, so
//      the MFMA fragment of V^T that covers 16 head dims x 32 positions is
//      one contiguous kilobyte. Inside a block, slot 8 g + j (g = 0..3)
//      holds position 4 g + j for j < 4 and 16 + 4 g + (j - 4) for j >= 4:
//      the order in which the attention kernel's probabilities leave its
//      score MFMAs (attention.hip), so P never has to be reshuffled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr int kVBlock = 32;

__host__ __device__ inline int v_slot(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }

// element offset of V[pos][d] inside one KV head's region
__host__ __device__ inline int64_t v_index(int64_t pos, int d, int hd) {
  return ((pos >> 5) * hd + d) * kVBlock + v_slot(static_cast<int>(pos & 31));
}

}  // namespace dg
