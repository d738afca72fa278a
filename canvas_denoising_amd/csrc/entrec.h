// Split-row softmax records of the sampler: a chunk of a logits row reduces to (m = max logit,
// Z = sum 2^u, A = sum u 2^u with u = (l - m) log2(e) / T, the lowest index of m), and records
// merge exactly (rescaled to the larger max), so a row's entropy H = ln Z - ln 2 A / Z and its
// argmax follow from any split of the row ([P3] "Inference mechanism": the entropy-bounded sampler;
// [P4] "Standard sampling settings"). Used by the sampler's partial pass and by the LM head when it
// produces the records of its vocabulary blocks itself.
#pragma once

#include "dg_common.h"

namespace dg {

struct Rec {
  float m;   // max raw logit (-inf when empty)
  float z;   // sum 2^u
  float a;   // sum u 2^u
  int idx;   // lowest index attaining m
};

// merge y into x; `c` = log2(e) / T. Deterministic for a fixed merge order.
__device__ inline void rec_merge(Rec& x, const Rec& y, float c) {
  if (y.z == 0.f) return;
  if (x.z == 0.f) { x = y; return; }
  const float m = fmaxf(x.m, y.m);
  const float dx = (x.m - m) * c, dy = (y.m - m) * c;
  const float sx = __builtin_amdgcn_exp2f(dx), sy = __builtin_amdgcn_exp2f(dy);
  const int idx = (x.m > y.m) ? x.idx : (y.m > x.m) ? y.idx : min(x.idx, y.idx);
  x.a = sx * (x.a + dx * x.z) + sy * (y.a + dy * y.z);
  x.z = x.z * sx + y.z * sy;
  x.m = m;
  x.idx = idx;
}

template <int CTRL>
__device__ inline Rec rec_dpp(const Rec& r) {
  return Rec{dpp_f32<CTRL>(r.m), dpp_f32<CTRL>(r.z), dpp_f32<CTRL>(r.a),
             static_cast<int>(dpp_u32<CTRL>(static_cast<uint32_t>(r.idx)))};
}
__device__ inline Rec rec_xrow16(const Rec& r) {
  return Rec{xrow16_f32(r.m), xrow16_f32(r.z), xrow16_f32(r.a),
             static_cast<int>(xrow16_u32(static_cast<uint32_t>(r.idx)))};
}
__device__ inline Rec rec_xrow32(const Rec& r) {
  return Rec{xrow32_f32(r.m), xrow32_f32(r.z), xrow32_f32(r.a),
             static_cast<int>(xrow32_u32(static_cast<uint32_t>(r.idx)))};
}

// Merge the records of all 64 lanes: six partner levels (dg_common.h), a fixed order per lane.
__device__ inline void rec_wave_merge(Rec& w, float c) {
  rec_merge(w, rec_dpp<kDppXor1>(w), c);
  rec_merge(w, rec_dpp<kDppXor2>(w), c);
  rec_merge(w, rec_dpp<kDppHalfMirror>(w), c);
  rec_merge(w, rec_dpp<kDppMirror>(w), c);
  rec_merge(w, rec_xrow16(w), c);
  rec_merge(w, rec_xrow32(w), c);
}

}  // namespace dg
