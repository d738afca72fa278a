// Fragment-tiled storage of the routed-expert matrices.
//
// A [R x K] weight matrix (rows = output features, K contiguous) is cut into
// tiles of 16 rows x 32 columns (512 elements). Inside a tile, "lane" l holds
// row l % 16 and the 8 consecutive columns 8 * (l / 16) .. +7 at elements
// 8 l .. 8 l + 7: exactly the MFMA operand fragment of one k-step (mfma.h), so
// one 16-byte (bf16) load per lane fetches a whole fragment and a wave reads
// one contiguous kilobyte.
//
// Tiles are grouped: a group holds `gr` consecutive 16-row blocks of each of
// `gw` matrices stored together, G = gr * gw tiles per k-step, ordered
// [group][k-tile][g] with g = which * gr + (row block % gr). The embedding
// matrix (the LM head's weights) uses gr = kVocabGroup, gw = 1; the routed
// experts use gate/up: gr = kGuBlocks, gw = 2 (blocks 2j, 2j+1 of the gate
// matrix next to the same blocks of the up matrix; gw = 1 without a gate),
// down: gr = kDownGroup, gw = 1. One workgroup streams one group: a
// contiguous run of G * K * 32 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr int kTileElems = 512;
constexpr int kVocabGroup = 2;  // 16-row blocks per tile group of the embedding (LM head) matrix
constexpr int kGuBlocks = 2;   // 16-feature blocks per tile group of an expert's gate/up matrices
constexpr int kDownGroup = 4;  // 16-row blocks per tile group of an expert's down matrix

// Physical element index of element (r, k) of matrix `which` (K columns).
__host__ __device__ inline int64_t tiled_index(int64_t r, int64_t k, int which, int64_t K, int gr, int gw) {
  const int64_t rb = r >> 4, kb = k >> 5;
  const int64_t group = rb / gr;
  const int g = which * gr + static_cast<int>(rb % gr);
  const int64_t tile = (group * (K >> 5) + kb) * (gr * gw) + g;
  const int lane = static_cast<int>(r & 15) + 16 * static_cast<int>((k & 31) >> 3);
  return tile * kTileElems + lane * 8 + (k & 7);
}

// Inverse of tiled_index: matrix, row and column of physical element p.
__host__ __device__ inline void tiled_coords(int64_t p, int64_t K, int gr, int gw, int* which, int64_t* r,
                                             int64_t* k) {
  const int G = gr * gw;
  const int64_t tile = p / kTileElems;
  const int in = static_cast<int>(p % kTileElems);
  const int lane = in >> 3;
  const int g = static_cast<int>(tile % G);
  const int64_t t2 = tile / G;
  const int64_t kt = K >> 5;
  const int64_t kb = t2 % kt, group = t2 / kt;
  *which = g / gr;
  *r = (group * gr + g % gr) * 16 + (lane & 15);
  *k = kb * 32 + (lane >> 4) * 8 + (in & 7);
}

}  // namespace dg

namespace dg {

// FP8 (E4M3) copies of the routed-expert matrices keep the tile order above
// with one byte per element, but pair the k-tiles: for k-tile pair p the
// 1 KiB block of tile g holds, for lane l at bytes 16 l .. 16 l + 15, the 8
// codes of lane l in k-tile 2p followed by its 8 codes in k-tile 2p + 1, so a
// 16-byte load per lane still moves a whole contiguous kilobyte per wave (two
// k-steps of B fragments). K must be a multiple of 64. Byte index of element
// (r, k) of matrix `which`:
__host__ __device__ inline int64_t fp8_tiled_index(int64_t r, int64_t k, int which, int64_t K, int gr, int gw) {
  const int64_t rb = r >> 4, kb = k >> 5;
  const int64_t group = rb / gr;
  const int g = which * gr + static_cast<int>(rb % gr);
  const int64_t block = (group * (K >> 6) + (kb >> 1)) * (gr * gw) + g;
  const int lane = static_cast<int>(r & 15) + 16 * static_cast<int>((k & 31) >> 3);
  return block * 1024 + lane * 16 + (kb & 1) * 8 + (k & 7);
}

}  // namespace dg
