// Model context of libdg: packed weight layout, KV cache, workspace carving and
// the host-side orchestration of the denoising step, the encoder pass (prompt
// prefill and block commit) and the native denoising loop.
//
// One denoising step ([P3] "Encoder-denoiser design", "Inference mechanism";
// [P4] "System architecture"):
//   self-conditioning from the previous step (probabilities rebuilt from the
//   sampler's row statistics, u = p E, sc = GeLU(u W1^T) W2^T),
//   x = E[canvas] + sc,
//   per layer: h = RMSNorm(x); [q k v] = h Wqkv^T with k, v written to the
//   cache scratch slots; o = attention (bidirectional); x += o Wo^T;
//   h = RMSNorm(x); router top-k; routed experts; shared expert;
//   x += shared + sum_k gate * expert (fixed order),
//   logits = RMSNorm(x) E^T.
// The encoder pass runs the same layers causally over prompt / block chunks.
#include <math.h>

#include <algorithm>
#include <string>
#include <vector>

#include "dg_common.h"
#include "gemm.h"
#include "prof.h"
#include "kvlayout.h"
#include "tiles.h"

namespace dg {

// kernels implemented in the .hip files
int embed(const void* emb, const int32_t* ids, const float* sc, float* x, int M, int D, int V, int dtype,
          hipStream_t s);
int rmsnorm(const float* x, void* h, int M, int D, float eps, int dtype, hipStream_t s);
int residual_norm(float* x, const float* part, int splits, const float* y, const float* slot_out,
                  const int32_t* slot_of, int k, void* h, int M, int D, float eps, int dtype, hipStream_t s,
                  const char* name, int y_planes = 1);
int transpose(const void* in, int64_t R, int64_t C, int gr, int gr_out, void* out, int dtype, hipStream_t s);
int sc_embed_splits(int N, int64_t K, int dtype);
int sc_embed(const void* logits, int64_t ldl, const float* stats, const float* temp, const void* Et, int M, int N,
             int64_t K, float* part, void* u, int dtype, hipStream_t s);
int zero_fill(void* p, size_t bytes, hipStream_t s);
int store_i32(int32_t* p, int32_t v, hipStream_t s);
int store_f32(float* p, float v, hipStream_t s);
int attention(const void* q, int64_t ldq, const void* kc, const void* vc, int64_t head_stride, int M, int Hq,
              int Hkv, int hd, int pos0, const int* pos_dev, int pos_max, int causal, float* part_o,
              float* part_ml, void* o, int64_t ldo, int dtype, hipStream_t s);
int attn_max_splits();
int attn_v_overrun();
int64_t attn_partial_rows(int M, int Hq, int Hkv);
int vocab_gemm(const void* h, int64_t ldh, const void* E, int M, int V, int D, void* logits, int64_t ldo, int dtype,
               hipStream_t s);
int vocab_gemm_stats(const void* h, int64_t ldh, const void* E, int M, int V, int D, void* logits, int64_t ldo,
                     const float* temp, void* recs, int dtype, hipStream_t s);
int vocab_blocks(int V);
int moe_route(const float* part, int splits, int M, int E, int k, int renorm, float* rlog, int32_t* sel,
              float* gate, int32_t* offsets, int32_t* perm, int32_t* slot_of, float* slot_gate, int32_t* tiles,
              hipStream_t s);
int moe_combine(float* x, const float* y, const float* slot_out, const int32_t* slot_of, int M, int D, int k,
                hipStream_t s);
int moe_experts(const void* h, int64_t ldh, const void* w_gu, const void* w_down, int E, int F, int D, int gated,
                const int32_t* offsets, const int32_t* perm, const float* slot_gate, void* act, float* out,
                int dtype, const ExpertsFp8* q8, const int32_t* tiles, int M, int k, hipStream_t s);
int rope_table(double theta, int hd, int64_t n_pos, float2* table, hipStream_t s);
int rope_apply(void* q, int64_t ldq, void* kc, int64_t kv_stride, int pos0, const int* pos_dev, int M, int Hq,
               int Hkv, int hd, const float2* table, int dtype, hipStream_t s);
int quantize_fp8(const void* src, int64_t src_stride, void* codes, int64_t code_stride, float* scales, int E, int R,
                 int K, int gr, int gw, hipStream_t s);
int launch_synth_normal(uint64_t seed, uint64_t tid, int64_t n, float sigma, int dtype, void* out, hipStream_t s);
int launch_synth_tiled(uint64_t seed, const uint64_t* tids, int64_t R, int64_t K, int gr, int gw, float sigma,
                       int dtype, void* out, hipStream_t s);
int pack_tiled(const void* src, int64_t R, int64_t K, int which, int gr, int gw, void* dst, int dtype,
               hipStream_t s);
size_t sample_workspace_bytes(int64_t rows, int64_t vocab);
int launch_sample_from_block_recs(const void* block_recs, int nblk, int rows, int vocab, float temp,
                                  const dg_sched& sc, int step, int block, int32_t* canvas, int32_t* pred,
                                  uint8_t* accept, float* entropy, float* row_stats, dg_stop_state* stop, void* ws,
                                  hipStream_t stream);
int launch_init_canvas(uint64_t seed, int block, int n, int vocab, int32_t* canvas, dg_stop_state* stop,
                       hipStream_t stream);
int launch_sample(const void* logits, int dtype, int rows, int vocab, float temp, const dg_sched& sc, int step,
                  int block, int32_t* canvas, int32_t* pred, uint8_t* accept, float* entropy, float* row_stats,
                  dg_stop_state* stop, void* ws, hipStream_t stream);
float temperature(const dg_sched& s, int step);
int check_sched(const dg_sched* s, int step);

#define DG_TRY(x)            \
  do {                       \
    int rc__ = (x);          \
    if (rc__ != DG_OK) return rc__; \
  } while (0)

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int esize(const dg_model_desc& d) { return d.dtype == DG_BF16 ? 2 : 4; }

// ------------------------------------------------------------ weight layout
struct WLayout {
  size_t embed = 0, embed_t = 0, sc1 = 0, sc2 = 0;
  std::vector<size_t> qkv, o, router, sh_gu, sh_down, ex_gu, ex_down;
  size_t total = 0;
};

static WLayout weight_layout(const dg_model_desc& d) {
  const size_t es = esize(d);
  size_t cur = 0;
  auto take = [&](int64_t elems) {
    const size_t off = cur;
    cur = align256(cur + static_cast<size_t>(elems) * es);
    return off;
  };
  WLayout L;
  const int64_t D = d.d_model, hd = d.head_dim;
  L.embed = take(static_cast<int64_t>(d.vocab) * D);
  L.embed_t = take(static_cast<int64_t>(d.vocab) * D);
  L.sc1 = take(static_cast<int64_t>(d.d_selfcond) * D);
  L.sc2 = take(static_cast<int64_t>(d.d_selfcond) * D);
  const int g = d.gated ? 2 : 1;
  for (int l = 0; l < d.n_layers; ++l) {
    L.qkv.push_back(take(static_cast<int64_t>(d.n_q_heads + 2 * d.n_kv_heads) * hd * D));
    L.o.push_back(take(static_cast<int64_t>(d.n_q_heads) * hd * D));
    L.router.push_back(take(static_cast<int64_t>(d.n_experts) * D));
    L.sh_gu.push_back(take(static_cast<int64_t>(g) * d.d_shared * D));
    L.sh_down.push_back(take(static_cast<int64_t>(d.d_shared) * D));
    L.ex_gu.push_back(take(static_cast<int64_t>(d.n_experts) * g * d.d_expert * D));
    L.ex_down.push_back(take(static_cast<int64_t>(d.n_experts) * d.d_expert * D));
  }
  L.total = cur;
  return L;
}

// FP8 copies of the routed experts, per layer: gate/up codes, down codes, their scales
struct Fp8Layout {
  std::vector<size_t> gu, dn, s_gu, s_dn;
  size_t total = 0;
};

static Fp8Layout fp8_layout(const dg_model_desc& d) {
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t off = cur;
    cur = align256(cur + bytes);
    return off;
  };
  const size_t E = d.n_experts, F = d.d_expert, D = d.d_model, gw = d.gated ? 2 : 1;
  Fp8Layout L;
  for (int l = 0; l < d.n_layers; ++l) {
    L.gu.push_back(take(E * gw * F * D));
    L.dn.push_back(take(E * D * F));
    L.s_gu.push_back(take(E * gw * F * 4));
    L.s_dn.push_back(take(E * D * 4));
  }
  L.total = cur;
  return L;
}

static int check_fp8_desc(const dg_model_desc* d) {
  if (d->dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "FP8 experts are built from a bf16 model");
  if (d->d_expert % 64 != 0 || d->d_model % 64 != 0)
    return fail(DG_ERR_UNSUPPORTED, "FP8 experts need d_expert and d_model multiples of 64");
  return DG_OK;
}

static int tensor_info(const dg_model_desc& d, const WLayout& L, int kind, int layer, int expert, size_t* off,
                       int64_t* rows, int64_t* cols) {
  const size_t es = esize(d);
  const int64_t D = d.d_model, hd = d.head_dim;
  const bool per_layer = kind >= DG_W_Q;
  if (per_layer && (layer < 0 || layer >= d.n_layers)) return fail(DG_ERR_INVALID, "layer out of range");
  if (kind >= DG_W_EX_GATE && (expert < 0 || expert >= d.n_experts)) return fail(DG_ERR_INVALID, "expert out of range");
  const int64_t F = d.d_expert, Fs = d.d_shared;
  const int64_t gu_stride = (d.gated ? 2 : 1) * F * D;
  switch (kind) {
    case DG_W_EMBED: *off = L.embed; *rows = d.vocab; *cols = D; break;
    case DG_W_EMBED_T: *off = L.embed_t; *rows = D; *cols = d.vocab; break;
    case DG_W_SC1: *off = L.sc1; *rows = d.d_selfcond; *cols = D; break;
    case DG_W_SC2: *off = L.sc2; *rows = D; *cols = d.d_selfcond; break;
    case DG_W_Q: *off = L.qkv[layer]; *rows = d.n_q_heads * hd; *cols = D; break;
    case DG_W_K: *off = L.qkv[layer] + d.n_q_heads * hd * D * es; *rows = d.n_kv_heads * hd; *cols = D; break;
    case DG_W_V:
      *off = L.qkv[layer] + (d.n_q_heads + d.n_kv_heads) * hd * D * es; *rows = d.n_kv_heads * hd; *cols = D;
      break;
    case DG_W_O: *off = L.o[layer]; *rows = D; *cols = d.n_q_heads * hd; break;
    case DG_W_ROUTER: *off = L.router[layer]; *rows = d.n_experts; *cols = D; break;
    case DG_W_SH_GATE:
      if (!d.gated) return fail(DG_ERR_INVALID, "ungated model has no gate weights");
      *off = L.sh_gu[layer]; *rows = Fs; *cols = D; break;
    case DG_W_SH_UP: *off = L.sh_gu[layer] + (d.gated ? Fs * D * es : 0); *rows = Fs; *cols = D; break;
    case DG_W_SH_DOWN: *off = L.sh_down[layer]; *rows = D; *cols = Fs; break;
    // routed experts: offset of the expert's fragment-tiled gate/up (or down) region
    case DG_W_EX_GATE:
      if (!d.gated) return fail(DG_ERR_INVALID, "ungated model has no gate weights");
      *off = L.ex_gu[layer] + expert * gu_stride * es; *rows = F; *cols = D; break;
    case DG_W_EX_UP: *off = L.ex_gu[layer] + expert * gu_stride * es; *rows = F; *cols = D; break;
    case DG_W_EX_DOWN: *off = L.ex_down[layer] + expert * D * F * es; *rows = D; *cols = F; break;
    default: return fail(DG_ERR_INVALID, "unknown weight kind");
  }
  return DG_OK;
}

// Tile grouping of the fragment-tiled kinds (tiles.h); false for row-major kinds.
static bool tiling_of(const dg_model_desc& d, int kind, int* which, int* gr, int* gw) {
  switch (kind) {
    case DG_W_EMBED: *which = 0; *gr = kVocabGroup; *gw = 1; return true;
    case DG_W_EX_GATE: *which = 0; *gr = kGuBlocks; *gw = 2; return true;
    case DG_W_EX_UP: *which = d.gated ? 1 : 0; *gr = kGuBlocks; *gw = d.gated ? 2 : 1; return true;
    case DG_W_EX_DOWN: *which = 0; *gr = kDownGroup; *gw = 1; return true;
    default: return false;
  }
}

int check_desc(const dg_model_desc* d) {
  if (d == nullptr) return fail(DG_ERR_INVALID, "desc is NULL");
  if (d->dtype != DG_BF16 && d->dtype != DG_F32) return fail(DG_ERR_INVALID, "dtype must be DG_BF16 or DG_F32");
  if (d->n_layers < 1) return fail(DG_ERR_SHAPE, "n_layers must be >= 1");
  if (d->canvas < 1 || d->canvas > 256) return fail(DG_ERR_UNSUPPORTED, "canvas must be in [1, 256]");
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return fail(DG_ERR_SHAPE, "n_q_heads must be a positive multiple of n_kv_heads");
  if (d->dtype == DG_BF16 && d->head_dim != 64 && d->head_dim != 128)
    return fail(DG_ERR_UNSUPPORTED, "bf16 head_dim must be 64 or 128");
  if (d->dtype == DG_F32 && (d->head_dim < 8 || d->head_dim > 128 || d->head_dim % 8 != 0))
    return fail(DG_ERR_UNSUPPORTED, "fp32 head_dim must be a multiple of 8 up to 128");
  const int64_t dims[] = {d->d_model, static_cast<int64_t>(d->n_q_heads) * d->head_dim, d->d_expert, d->d_shared,
                          d->d_selfcond, d->vocab};
  for (int64_t v : dims)
    if (v < 64 || v % 64 != 0) return fail(DG_ERR_UNSUPPORTED, "d_model, q width, FFN widths and vocab must be multiples of 64");
  if (d->d_model % (16 * kDownGroup) != 0) return fail(DG_ERR_UNSUPPORTED, "d_model must be a multiple of 64");
  if (d->n_experts < 1 || d->n_experts > 256) return fail(DG_ERR_UNSUPPORTED, "n_experts must be in [1, 256]");
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts) return fail(DG_ERR_UNSUPPORTED, "top_k must be in [1, min(16, n_experts)]");
  if (!(d->rms_eps >= 0.f) || !isfinite(d->rms_eps)) return fail(DG_ERR_INVALID, "rms_eps must be finite and >= 0");
  if (d->gated != 0 && d->gated != 1) return fail(DG_ERR_INVALID, "gated must be 0 or 1");
  if (!(d->rope_theta >= 0.f) || !isfinite(d->rope_theta)) return fail(DG_ERR_INVALID, "rope_theta must be finite and >= 0");
  if (d->prefill_rows != 0 && (d->prefill_rows < d->canvas || d->prefill_rows > 4096))
    return fail(DG_ERR_UNSUPPORTED, "prefill_rows must be 0 or in [canvas, 4096]");
  if (d->prefill_rows > 256 && d->n_experts > 128)
    return fail(DG_ERR_UNSUPPORTED, "prefill chunks of more than 256 rows need n_experts <= 128");
  return DG_OK;
}

// a captured denoising step body and the caller's buffers it was captured for (the committed KV
// length and the self-conditioning temperature are read on the device, so they are not part of it)
struct StepGraph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  const int32_t* canvas = nullptr;
  const void* logits = nullptr;
  const void* prev_logits = nullptr;
  const float* prev_stats = nullptr;
};

// ----------------------------------------------------------- workspace layout
struct WsLayout {
  size_t x, h, q, o, part_o, part_ml, rlog, sel, gate, offsets, perm, slot_of, slot_gate, act, slot_out, sh_act,
      sc, u, sc_hid, scpart, gpart, gpart_aux, y_sh, canvas, pred, accept, entropy, row_stats, stop, samp, rope,
      tiles, len_dev, sc_temp, lm_temp, vrecs, total;
  int64_t gpart_floats;
  int64_t sel_layer;  // elements between the layers' expert choices (and gates)
};

// rows of one layer pass: a canvas, or a prefill / commit chunk
static int64_t pass_rows(const dg_model_desc& d) { return std::max<int64_t>(d.canvas, d.prefill_rows); }

static WsLayout ws_layout(const dg_model_desc& d, int64_t capacity) {
  const size_t es = esize(d);
  const int64_t D = d.d_model, QW = static_cast<int64_t>(d.n_q_heads) * d.head_dim;
  const int64_t C = pass_rows(d);  // activation rows (the canvas-only buffers below use d.canvas)
  const int64_t CK = C * d.top_k;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t off = cur;
    cur = align256(cur + bytes);
    return off;
  };
  WsLayout w;
  w.x = take(C * D * 4);
  w.h = take(C * D * es);
  w.q = take(C * QW * es);
  w.o = take(C * QW * es);
  int64_t prow = 0;  // splits x rows of the attention partials, over every pass size up to C
  for (int m = 1; m <= C; ++m) prow = std::max(prow, attn_partial_rows(m, d.n_q_heads, d.n_kv_heads));
  w.part_o = take(static_cast<size_t>(prow) * d.n_q_heads * d.head_dim * 4);
  w.part_ml = take(static_cast<size_t>(prow) * d.n_q_heads * 2 * 4);
  w.rlog = take(C * d.n_experts * 4);
  // the expert choices and gates of every layer of the last pass (layer l at l * sel_layer)
  w.sel_layer = CK;
  w.sel = take(static_cast<size_t>(d.n_layers) * CK * 4);
  w.gate = take(static_cast<size_t>(d.n_layers) * CK * 4);
  w.offsets = take((2 * d.n_experts + 1) * 4);  // slot offsets, then the experts by token count
  w.perm = take(CK * 4);
  w.slot_of = take(CK * 4);
  w.slot_gate = take(CK * 4);
  w.act = take(CK * d.d_expert * es);
  w.slot_out = take(CK * D * 4);
  w.sh_act = take(C * d.d_shared * es);
  // canvas-only buffers: self-conditioning, split-K scratch, sampler state
  const int64_t Cc = d.canvas;
  w.sc = take(Cc * D * 4);
  w.u = take(Cc * D * es);
  w.sc_hid = take(Cc * d.d_selfcond * es);
  w.scpart = take(static_cast<size_t>(sc_embed_splits(static_cast<int>(D), d.vocab, d.dtype)) * Cc * D * 4);
  w.gpart_floats = 32 * Cc * std::max<int64_t>(std::max<int64_t>(D, d.d_selfcond), d.n_experts);
  w.gpart = take(w.gpart_floats * 4);
  w.gpart_aux = take(w.gpart_floats * 4);  // split-K scratch of the second stream
  w.y_sh = take(C * D * 4);
  w.canvas = take(Cc * 4);
  w.pred = take(Cc * 4);
  w.accept = take(Cc);
  w.entropy = take(Cc * 4);
  w.row_stats = take(Cc * 8);
  w.stop = take(sizeof(dg_stop_state));
  w.samp = take(sample_workspace_bytes(Cc, d.vocab));
  // rotary embedding: (cos, sin) per cache position and frequency
  w.rope = take(d.rope_theta > 0.f ? static_cast<size_t>(capacity) * (d.head_dim / 2) * 8 : 0);
  w.tiles = take((2 + CK / 128 + d.n_experts + 8) * 4);  // token-tile list of a chunk
  w.len_dev = take(4);   // int32: the committed KV length, as the denoising step reads it
  w.sc_temp = take(4);   // float: the temperature of the self-conditioning distribution
  w.lm_temp = take(4);   // float: the temperature of the LM head's sampler records
  w.vrecs = take(static_cast<size_t>(Cc) * vocab_blocks(static_cast<int>(d.vocab)) * 16);  // [canvas][blocks] records
  w.total = cur;
  return w;
}

}  // namespace dg

struct dg_ctx {
  dg_model_desc d;
  char* w;
  char* kv;
  int64_t cap;
  int64_t len;
  char* ws;
  size_t ws_bytes;
  dg::WLayout wl;
  dg::WsLayout wsl;
  // second stream: the shared expert runs beside the routed experts (fork / join events)
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // FP8 routed experts in use (dg_ctx_use_expert_fp8), else null
  const char* fp8 = nullptr;
  dg::Fp8Layout fl;
  // graph replay of the denoising step body ([0]: without self-conditioning, [1]: with)
  hipStream_t cap_stream = nullptr;
  bool use_graphs = true;
  dg::StepGraph graphs[2];
  // the LM head also folds its logits into the sampler's split-row records at this schedule's
  // temperature (dg_ctx_fuse_sampler_stats), so the sampler need not read the logits again
  bool fuse_stats = false;
  dg_sched fuse_sched{};
  int last_layer = 0;  // layer of the last routing (DG_BUF_SEL / DG_BUF_GATE)
  int64_t captures = 0;  // step graphs captured so far
  // dg_generate_block's read-back of the stop state: one pinned host slot and one event per step in
  // flight
  static constexpr int kStopSlots = 16;
  dg_stop_state* stop_host = nullptr;
  hipEvent_t stop_ev[kStopSlots] = {};
};

namespace dg {

template <typename P> static P* wsp(dg_ctx* c, size_t off) { return reinterpret_cast<P*>(c->ws + off); }
static void* wp(dg_ctx* c, size_t off) { return c->w + off; }

static void* kv_k(dg_ctx* c, int l) {
  const size_t es = esize(c->d);
  return c->kv + static_cast<size_t>(l) * c->d.n_kv_heads * c->cap * c->d.head_dim * es;
}
static void* kv_v(dg_ctx* c, int l) {
  const size_t es = esize(c->d);
  return c->kv + static_cast<size_t>(c->d.n_layers + l) * c->d.n_kv_heads * c->cap * c->d.head_dim * es;
}

#ifndef DG_QKV_SPLIT
#define DG_QKV_SPLIT 0
#endif
constexpr bool kQkvSplit = DG_QKV_SPLIT;   // split-K for the fused QKV projection (reduce applies the cache epilogue)

static int run_gemm(dg_ctx* c, GemmArgs g, hipStream_t s, const char* name, bool allow_split, bool aux = false) {
  const int splits = gemm_pick_splits(g.M, g.N, g.K, c->d.dtype, c->wsl.gpart_floats, allow_split);
  g.part = wsp<float>(c, aux ? c->wsl.gpart_aux : c->wsl.gpart);
  return gemm(g, c->d.dtype, splits, s, name);
}

// row kernels can hold a residual row in registers up to this width (residual_norm)
#ifndef DG_FUSED_NORM
#define DG_FUSED_NORM 1
#endif
// the shared expert's down projection leaves its split-K partials to the combine instead of reducing
// them in a kernel of its own on the second stream
#ifndef DG_SHARED_DEFER
#define DG_SHARED_DEFER 1
#endif
constexpr bool kSharedDeferReduce = DG_SHARED_DEFER;
static bool fused_norm_ok(const dg_model_desc& d) {
  return DG_FUSED_NORM && d.d_model % 4 == 0 && d.d_model <= 3072;
}

// One layer over M rows of the residual stream x placed at cache positions pos0 .. pos0+M-1 (pos_dev
// non-null: pos0 is the committed length as the device holds it, so a captured launch serves any).
// On entry h = RMSNorm(x); on exit x is the layer's output and h = RMSNorm(x) again (the next
// layer's input norm, or the final norm before the LM head): every residual update is fused with
// the norm that follows it. `kv_only` stops after the K/V projection (last encoder layer).
static int layer_forward(dg_ctx* c, int l, float* x, int M, int pos0, const int* pos_dev, bool causal, bool kv_only,
                         hipStream_t s) {
  const dg_model_desc& d = c->d;
  const WsLayout& w = c->wsl;
  const int D = d.d_model, hd = d.head_dim, QW = d.n_q_heads * hd;
  const bool fused = fused_norm_ok(d);
  void* h = wsp<void>(c, w.h);
  {
    GemmArgs g;
    g.A = h; g.lda = D;
    g.B = wp(c, c->wl.qkv[l]); g.ldb = D;
    g.M = M; g.N = (d.n_q_heads + 2 * d.n_kv_heads) * hd; g.K = D;
    g.epi = EPI_QKV; g.out = wsp<void>(c, w.q); g.ldo = QW;
    g.q_cols = kv_only ? 0 : QW; g.head_dim = hd; g.n_kv = d.n_kv_heads; g.pos0 = pos0;
    g.kv_head_stride = c->cap * hd; g.kcache = kv_k(c, l); g.vcache = kv_v(c, l); g.pos_dev = pos_dev;
    if (kv_only) {  // only the K/V rows of the fused projection
      g.B = static_cast<const char*>(g.B) + static_cast<size_t>(QW) * D * esize(d);
      g.N = 2 * d.n_kv_heads * hd;
    }
    DG_TRY(run_gemm(c, g, s, "qkv_proj", kQkvSplit));
  }
  if (d.rope_theta > 0.f)
    DG_TRY(rope_apply(kv_only ? nullptr : wsp<void>(c, w.q), QW, kv_k(c, l), c->cap * hd, pos0, pos_dev, M,
                      d.n_q_heads, d.n_kv_heads, hd, wsp<float2>(c, w.rope), d.dtype, s));
  if (kv_only) return DG_OK;
  DG_TRY(attention(wsp<void>(c, w.q), QW, kv_k(c, l), kv_v(c, l), c->cap * hd, M, d.n_q_heads, d.n_kv_heads, hd,
                   pos0, pos_dev, static_cast<int>(c->cap) - M, causal ? 1 : 0, wsp<float>(c, w.part_o),
                   wsp<float>(c, w.part_ml), wsp<void>(c, w.o), QW, d.dtype, s));
  {
    GemmArgs g;
    g.A = wsp<void>(c, w.o); g.lda = QW;
    g.B = wp(c, c->wl.o[l]); g.ldb = QW;
    g.M = M; g.N = D; g.K = QW;
    g.epi = EPI_ADD_F32; g.out = x; g.ldo = D;
    int splits = 1;
    g.defer_reduce = fused;
    g.splits_out = &splits;
    DG_TRY(run_gemm(c, g, s, "o_proj", true));
    // x += (sum of the split partials, if the GEMM left them); h = RMSNorm(x)
    if (fused)
      DG_TRY(residual_norm(x, wsp<float>(c, w.gpart), splits > 1 ? splits : 0, nullptr, nullptr, nullptr, 0, h, M,
                           D, d.rms_eps, d.dtype, s, splits > 1 ? "o_reduce_norm" : "rmsnorm"));
    else
      DG_TRY(rmsnorm(x, h, M, D, d.rms_eps, d.dtype, s));
  }
  // the shared expert: h -> y_sh, or (fused combine) its down projection's split-K partials, which
  // the combine sums as the shared term (sh_planes of them, in order)
  int sh_planes = 1;
  auto shared = [&](hipStream_t st, bool on_aux) -> int {
    {
      GemmArgs g;
      g.A = h; g.lda = D;
      g.B = wp(c, c->wl.sh_gu[l]); g.ldb = D;
      g.M = M; g.N = (d.gated ? 2 : 1) * d.d_shared; g.K = D;
      g.epi = d.gated ? EPI_GEGLU : EPI_GELU; g.pair_f = d.d_shared;
      g.out = wsp<void>(c, w.sh_act); g.ldo = d.d_shared;
      DG_TRY(run_gemm(c, g, st, "shared_gateup", false, on_aux));
    }
    GemmArgs g;
    g.A = wsp<void>(c, w.sh_act); g.lda = d.d_shared;
    g.B = wp(c, c->wl.sh_down[l]); g.ldb = d.d_shared;
    g.M = M; g.N = D; g.K = d.d_shared;
    g.epi = EPI_STORE_F32; g.out = wsp<float>(c, w.y_sh); g.ldo = D;
    g.defer_reduce = fused && kSharedDeferReduce;
    g.splits_out = &sh_planes;
    return run_gemm(c, g, st, "shared_down", true, on_aux);
  };
  // The shared expert runs on the second stream beside the routing and the routed experts (both
  // only read h; each stream has its own split-K scratch). The fork point is here, right after the
  // norm, but its launches are enqueued after the routed experts': a replayed graph keeps the
  // first-captured child of a node on that node's hardware queue, so this order keeps the whole
  // routing -> experts -> combine chain on one queue (a change of queue costs several microseconds
  // on the critical path; measured 70.9-73.0 vs 74.2-74.6 steps/s for the 30-layer loop).
  DG_HIP(hipEventRecord(c->ev_fork, s));
  {
    // router logits as split-k partials (summed in order by the routing kernel)
    GemmArgs g;
    g.A = h; g.lda = D;
    g.B = wp(c, c->wl.router[l]); g.ldb = D;
    g.M = M; g.N = d.n_experts; g.K = D;
    g.epi = EPI_STORE_F32; g.out = wsp<void>(c, w.rlog); g.ldo = d.n_experts;
    int splits = 1;
    g.defer_reduce = true;
    g.splits_out = &splits;
    DG_TRY(run_gemm(c, g, s, "router", true));
    c->last_layer = l;
    DG_TRY(moe_route(splits > 1 ? wsp<float>(c, w.gpart) : wsp<float>(c, w.rlog), splits, M, d.n_experts, d.top_k,
                     d.renorm_gates, wsp<float>(c, w.rlog), wsp<int32_t>(c, w.sel) + l * w.sel_layer,
                     wsp<float>(c, w.gate) + l * w.sel_layer,
                     wsp<int32_t>(c, w.offsets), wsp<int32_t>(c, w.perm), wsp<int32_t>(c, w.slot_of),
                     wsp<float>(c, w.slot_gate), M > 256 ? wsp<int32_t>(c, w.tiles) : nullptr, s));
  }
  ExpertsFp8 q8;
  if (c->fp8) {
    q8.gu = reinterpret_cast<const uint8_t*>(c->fp8 + c->fl.gu[l]);
    q8.dn = reinterpret_cast<const uint8_t*>(c->fp8 + c->fl.dn[l]);
    q8.s_gu = reinterpret_cast<const float*>(c->fp8 + c->fl.s_gu[l]);
    q8.s_dn = reinterpret_cast<const float*>(c->fp8 + c->fl.s_dn[l]);
  }
  DG_TRY(moe_experts(h, D, wp(c, c->wl.ex_gu[l]), wp(c, c->wl.ex_down[l]), d.n_experts, d.d_expert, D, d.gated,
                     wsp<int32_t>(c, w.offsets), wsp<int32_t>(c, w.perm), wsp<float>(c, w.slot_gate),
                     wsp<void>(c, w.act), wsp<float>(c, w.slot_out), d.dtype, c->fp8 ? &q8 : nullptr,
                     M > 256 ? wsp<int32_t>(c, w.tiles) : nullptr, M, d.top_k, s));
  DG_HIP(hipStreamWaitEvent(c->aux, c->ev_fork, 0));
  DG_TRY(shared(c->aux, true));
  DG_HIP(hipEventRecord(c->ev_join, c->aux));
  // join, then x += shared + sum of the token's gated expert outputs (fixed order); h = RMSNorm(x)
  DG_HIP(hipStreamWaitEvent(s, c->ev_join, 0));
  if (fused) {
    const bool planes = kSharedDeferReduce && sh_planes > 1;
    return residual_norm(x, nullptr, 0, planes ? wsp<float>(c, w.gpart_aux) : wsp<float>(c, w.y_sh),
                         wsp<float>(c, w.slot_out), wsp<int32_t>(c, w.slot_of), d.top_k, h, M, D, d.rms_eps, d.dtype,
                         s, "combine_norm", planes ? sh_planes : 1);
  }
  DG_TRY(moe_combine(x, wsp<float>(c, w.y_sh), wsp<float>(c, w.slot_out), wsp<int32_t>(c, w.slot_of), M, D,
                     d.top_k, s));
  return rmsnorm(x, h, M, D, d.rms_eps, d.dtype, s);
}

static int encode(dg_ctx* c, const int32_t* ids, int n, hipStream_t s) {
  const dg_model_desc& d = c->d;
  float* x = wsp<float>(c, c->wsl.x);
  const int chunk = static_cast<int>(pass_rows(d));
  for (int c0 = 0; c0 < n; c0 += chunk) {
    const int M = std::min(chunk, n - c0);
    DG_TRY(embed(wp(c, c->wl.embed), ids + c0, nullptr, x, M, d.d_model, d.vocab, d.dtype, s));
    DG_TRY(rmsnorm(x, wsp<void>(c, c->wsl.h), M, d.d_model, d.rms_eps, d.dtype, s));
    for (int l = 0; l < d.n_layers; ++l)
      DG_TRY(layer_forward(c, l, x, M, static_cast<int>(c->len), nullptr, true, l == d.n_layers - 1, s));
    c->len += M;
  }
  // the denoising step reads the committed length on the device
  return store_i32(wsp<int32_t>(c, c->wsl.len_dev), static_cast<int32_t>(c->len), s);
}

// A denoising step: self-conditioning from the previous step's logits and row statistics (when
// prev_logits is set; the tempered probabilities are formed inside the P E product with the
// temperature the device holds), the embedding, the layers and the LM head. Its launches depend
// only on the caller's pointers and on whether self-conditioning is on (the committed KV length and
// the temperature are read on the device), so it is captured once and replayed.
static int denoise_body(dg_ctx* c, const int32_t* canvas, const void* prev_logits, const float* prev_stats,
                        void* logits, hipStream_t s) {
  const dg_model_desc& d = c->d;
  const WsLayout& w = c->wsl;
  const int C = d.canvas, D = d.d_model;
  float* x = wsp<float>(c, w.x);
  const float* sc = nullptr;
  if (prev_logits) {
    // u = P E: P [C x V] the tempered distribution of the previous logits (formed in the kernel),
    // E^T [D x V] tiled like the embedding
    DG_TRY(sc_embed(prev_logits, d.vocab, prev_stats, wsp<float>(c, w.sc_temp), wp(c, c->wl.embed_t), C, D,
                    d.vocab, wsp<float>(c, w.scpart), wsp<void>(c, w.u), d.dtype, s));
    {
      GemmArgs g;
      g.A = wsp<void>(c, w.u); g.lda = D;
      g.B = wp(c, c->wl.sc1); g.ldb = D;
      g.M = C; g.N = d.d_selfcond; g.K = D;
      g.epi = EPI_GELU; g.out = wsp<void>(c, w.sc_hid); g.ldo = d.d_selfcond;
      DG_TRY(run_gemm(c, g, s, "sc_ffn1", true));
    }
    {
      GemmArgs g;
      g.A = wsp<void>(c, w.sc_hid); g.lda = d.d_selfcond;
      g.B = wp(c, c->wl.sc2); g.ldb = d.d_selfcond;
      g.M = C; g.N = D; g.K = d.d_selfcond;
      g.epi = EPI_STORE_F32; g.out = wsp<void>(c, w.sc); g.ldo = D;
      DG_TRY(run_gemm(c, g, s, "sc_ffn2", true));
    }
    sc = wsp<float>(c, w.sc);
  }
  void* h = wsp<void>(c, w.h);
  DG_TRY(embed(wp(c, c->wl.embed), canvas, sc, x, C, D, d.vocab, d.dtype, s));
  DG_TRY(rmsnorm(x, h, C, D, d.rms_eps, d.dtype, s));
  const int* pos_dev = wsp<int32_t>(c, w.len_dev);
  for (int l = 0; l < d.n_layers; ++l)  // each layer leaves h = RMSNorm(its output)
    DG_TRY(layer_forward(c, l, x, C, static_cast<int>(c->len), pos_dev, false, false, s));
  if (c->fuse_stats)
    return vocab_gemm_stats(h, D, wp(c, c->wl.embed), C, d.vocab, D, logits, d.vocab, wsp<float>(c, w.lm_temp),
                            wsp<void>(c, w.vrecs), d.dtype, s);
  return vocab_gemm(h, D, wp(c, c->wl.embed), C, d.vocab, D, logits, d.vocab, d.dtype, s);
}

static void drop_graph(StepGraph& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.graph) (void)hipGraphDestroy(g.graph);
  g = StepGraph{};
}

// Replay of denoise_body as a HIP graph: ~500 dependent launches per step cost launch gaps that
// a graph removes. Captured on the context's own stream (the caller's may be the legacy default
// stream, which cannot capture; the second stream joins through the fork event), launched on s.
// While per-kernel profiling is on, steps run eagerly so every launch records its events.
static int denoise_graphed(dg_ctx* c, const int32_t* canvas, const void* prev_logits, const float* prev_stats,
                           void* logits, hipStream_t s) {
  if (prof_on() || !c->use_graphs) return denoise_body(c, canvas, prev_logits, prev_stats, logits, s);
  StepGraph& g = c->graphs[prev_logits ? 1 : 0];
  if (!(g.exec && g.canvas == canvas && g.logits == logits && g.prev_logits == prev_logits &&
        g.prev_stats == prev_stats)) {
    drop_graph(g);
    DG_HIP(hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    const int rc = denoise_body(c, canvas, prev_logits, prev_stats, logits, c->cap_stream);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cap_stream, &graph);
    if (rc != DG_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return hip_check(e, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (ie != hipSuccess) {
      (void)hipGraphDestroy(graph);
      return hip_check(ie, "hipGraphInstantiate");
    }
    g.graph = graph;
    g.exec = exec;
    g.canvas = canvas;
    g.logits = logits;
    g.prev_logits = prev_logits;
    g.prev_stats = prev_stats;
    ++c->captures;
  }
  DG_HIP(hipGraphLaunch(g.exec, s));
  return DG_OK;
}

static int denoise(dg_ctx* c, int step, const int32_t* canvas, const void* prev_logits, const float* prev_stats,
                   float prev_t, void* logits, hipStream_t s) {
  if (prev_logits != nullptr) DG_TRY(store_f32(wsp<float>(c, c->wsl.sc_temp), prev_t, s));
  if (c->fuse_stats) DG_TRY(store_f32(wsp<float>(c, c->wsl.lm_temp), temperature(c->fuse_sched, step), s));
  return denoise_graphed(c, canvas, prev_logits, prev_stats, logits, s);
}

// two schedules give every step the same temperature
static bool same_temperatures(const dg_sched& a, const dg_sched& b) {
  return a.max_steps == b.max_steps && a.t_start == b.t_start && a.t_end == b.t_end;
}

static int check_ctx(const dg_ctx* c) {
  if (c == nullptr) return fail(DG_ERR_INVALID, "ctx is NULL");
  return DG_OK;
}

}  // namespace dg

using namespace dg;

extern "C" {

size_t dg_weights_bytes(const dg_model_desc* desc) {
  if (check_desc(desc) != DG_OK) return 0;
  return weight_layout(*desc).total;
}

int dg_weight_tensor(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert, size_t* offset,
                     int64_t* rows, int64_t* cols) {
  DG_TRY(check_desc(desc));
  if (!offset || !rows || !cols) return fail(DG_ERR_INVALID, "output pointers required");
  const WLayout L = weight_layout(*desc);
  return tensor_info(*desc, L, kind, layer, expert, offset, rows, cols);
}

int dg_load_weight(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert, const void* d_src,
                   void* d_weights, void* stream) {
  DG_TRY(check_desc(desc));
  if (!d_src || !d_weights) return fail(DG_ERR_INVALID, "d_src and d_weights are required");
  if (kind == DG_W_EMBED_T) return fail(DG_ERR_INVALID, "DG_W_EMBED_T is derived by dg_prepare_weights");
  const WLayout L = weight_layout(*desc);
  size_t off;
  int64_t r, c;
  DG_TRY(tensor_info(*desc, L, kind, layer, expert, &off, &r, &c));
  char* dst = static_cast<char*>(d_weights) + off;
  hipStream_t s = as_stream(stream);
  int which, gr, gw;
  if (tiling_of(*desc, kind, &which, &gr, &gw)) return pack_tiled(d_src, r, c, which, gr, gw, dst, desc->dtype, s);
  DG_HIP(hipMemcpyAsync(dst, d_src, static_cast<size_t>(r * c) * esize(*desc), hipMemcpyDeviceToDevice, s));
  return DG_OK;
}

int dg_prepare_weights(const dg_model_desc* desc, void* d_weights, void* stream) {
  DG_TRY(check_desc(desc));
  if (!d_weights) return fail(DG_ERR_INVALID, "d_weights is NULL");
  const WLayout L = weight_layout(*desc);
  char* w = static_cast<char*>(d_weights);
  return transpose(w + L.embed, desc->vocab, desc->d_model, kVocabGroup, kVocabGroup, w + L.embed_t, desc->dtype,
                   as_stream(stream));
}

size_t dg_expert_fp8_bytes(const dg_model_desc* desc) {
  if (check_desc(desc) != DG_OK || check_fp8_desc(desc) != DG_OK) return 0;
  return fp8_layout(*desc).total;
}

int dg_expert_fp8_tensor(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert, size_t* code_offset,
                         size_t* scale_offset) {
  DG_TRY(check_desc(desc));
  DG_TRY(check_fp8_desc(desc));
  if (!code_offset || !scale_offset) return fail(DG_ERR_INVALID, "output pointers are NULL");
  const dg_model_desc& d = *desc;
  if (layer < 0 || layer >= d.n_layers) return fail(DG_ERR_INVALID, "layer out of range");
  if (expert < 0 || expert >= d.n_experts) return fail(DG_ERR_INVALID, "expert out of range");
  if (kind != DG_W_EX_UP && kind != DG_W_EX_DOWN && !(kind == DG_W_EX_GATE && d.gated))
    return fail(DG_ERR_INVALID, "kind must be a routed-expert matrix of this model");
  const Fp8Layout L = fp8_layout(d);
  const size_t E = expert, F = d.d_expert, D = d.d_model, gw = d.gated ? 2 : 1;
  if (kind == DG_W_EX_DOWN) {
    *code_offset = L.dn[layer] + E * D * F;
    *scale_offset = L.s_dn[layer] + E * D * 4;
  } else {
    const size_t which = (kind == DG_W_EX_UP && d.gated) ? 1 : 0;
    *code_offset = L.gu[layer] + E * gw * F * D;
    *scale_offset = L.s_gu[layer] + (E * gw + which) * F * 4;
  }
  return DG_OK;
}

int dg_quantize_experts_fp8(const dg_model_desc* desc, const void* d_weights, void* d_fp8, void* stream) {
  DG_TRY(check_desc(desc));
  DG_TRY(check_fp8_desc(desc));
  if (!d_weights || !d_fp8) return fail(DG_ERR_INVALID, "d_weights and d_fp8 are required");
  if (reinterpret_cast<uintptr_t>(d_weights) % 256 != 0 || reinterpret_cast<uintptr_t>(d_fp8) % 256 != 0)
    return fail(DG_ERR_INVALID, "device buffers must be 256-byte aligned");
  const dg_model_desc& d = *desc;
  const WLayout W = weight_layout(d);
  const Fp8Layout L = fp8_layout(d);
  const char* w = static_cast<const char*>(d_weights);
  char* q = static_cast<char*>(d_fp8);
  hipStream_t s = as_stream(stream);
  const int64_t F = d.d_expert, D = d.d_model, gw = d.gated ? 2 : 1;
  for (int l = 0; l < d.n_layers; ++l) {
    DG_TRY(quantize_fp8(w + W.ex_gu[l], gw * F * D, q + L.gu[l], gw * F * D, reinterpret_cast<float*>(q + L.s_gu[l]),
                        d.n_experts, static_cast<int>(F), static_cast<int>(D), kGuBlocks, static_cast<int>(gw), s));
    DG_TRY(quantize_fp8(w + W.ex_down[l], D * F, q + L.dn[l], D * F, reinterpret_cast<float*>(q + L.s_dn[l]),
                        d.n_experts, static_cast<int>(D), static_cast<int>(F), kDownGroup, 1, s));
  }
  return DG_OK;
}

int dg_synth_fill_weights(const dg_model_desc* desc, uint64_t seed, float sigma, void* d_weights, void* stream) {
  DG_TRY(check_desc(desc));
  if (!d_weights) return fail(DG_ERR_INVALID, "d_weights is NULL");
  if (!isfinite(sigma) || sigma < 0.f) return fail(DG_ERR_INVALID, "sigma must be finite and >= 0");
  const dg_model_desc& d = *desc;
  const WLayout L = weight_layout(d);
  hipStream_t s = as_stream(stream);
  char* w = static_cast<char*>(d_weights);
  auto fill = [&](int kind, int layer, int expert, uint64_t tid) -> int {
    size_t off;
    int64_t r, cl;
    DG_TRY(tensor_info(d, L, kind, layer, expert, &off, &r, &cl));
    return launch_synth_normal(seed, tid, r * cl, sigma, d.dtype, w + off, s);
  };
  const uint64_t kLayer = 1ull << 20, kExpert = 1ull << 32;
  {
    const uint64_t tid[1] = {1};
    DG_TRY(launch_synth_tiled(seed, tid, d.vocab, d.d_model, kVocabGroup, 1, sigma, d.dtype, w + L.embed, s));
  }
  DG_TRY(fill(DG_W_SC1, 0, 0, 2));
  DG_TRY(fill(DG_W_SC2, 0, 0, 3));
  for (int l = 0; l < d.n_layers; ++l) {
    const uint64_t lb = kLayer + 64ull * l;
    DG_TRY(fill(DG_W_Q, l, 0, lb + 0));
    DG_TRY(fill(DG_W_K, l, 0, lb + 1));
    DG_TRY(fill(DG_W_V, l, 0, lb + 2));
    DG_TRY(fill(DG_W_O, l, 0, lb + 3));
    DG_TRY(fill(DG_W_ROUTER, l, 0, lb + 4));
    if (d.gated) DG_TRY(fill(DG_W_SH_GATE, l, 0, lb + 5));
    DG_TRY(fill(DG_W_SH_UP, l, 0, lb + 6));
    DG_TRY(fill(DG_W_SH_DOWN, l, 0, lb + 7));
    const size_t es = esize(d);
    for (int e = 0; e < d.n_experts; ++e) {
      const uint64_t eb = kExpert + 8ull * (1024ull * l + e);
      const uint64_t gu_tids[2] = {d.gated ? eb + 0 : eb + 1, eb + 1};
      const size_t gu_off = L.ex_gu[l] + static_cast<size_t>(e) * (d.gated ? 2 : 1) * d.d_expert * d.d_model * es;
      DG_TRY(launch_synth_tiled(seed, gu_tids, d.d_expert, d.d_model, kGuBlocks, d.gated ? 2 : 1, sigma, d.dtype,
                                w + gu_off, s));
      const uint64_t dn_tid[1] = {eb + 2};
      const size_t dn_off = L.ex_down[l] + static_cast<size_t>(e) * d.d_model * d.d_expert * es;
      DG_TRY(launch_synth_tiled(seed, dn_tid, d.d_model, d.d_expert, kDownGroup, 1, sigma, d.dtype, w + dn_off, s));
    }
  }
  return transpose(w + L.embed, d.vocab, d.d_model, kVocabGroup, kVocabGroup, w + L.embed_t, d.dtype, s);
}

size_t dg_kv_bytes(const dg_model_desc* desc, int64_t capacity) {
  if (check_desc(desc) != DG_OK || capacity < 0) return 0;
  // K and V of every layer and head, then a tail that the attention kernel's whole-stage V copies
  // may read (never write) past the last head's blocks
  const size_t kv = 2ull * desc->n_layers * desc->n_kv_heads * static_cast<size_t>(capacity) * desc->head_dim;
  return (kv + static_cast<size_t>(attn_v_overrun()) * desc->head_dim) * esize(*desc);
}

size_t dg_workspace_size(const dg_model_desc* desc, int64_t capacity) {
  if (check_desc(desc) != DG_OK || capacity < 0) return 0;
  return ws_layout(*desc, capacity).total;
}

int dg_ctx_create(const dg_model_desc* desc, void* d_weights, void* d_kv, int64_t capacity, void* d_workspace,
                  size_t ws_bytes, dg_ctx** out) {
  DG_TRY(check_desc(desc));
  if (!out) return fail(DG_ERR_INVALID, "out is NULL");
  if (!d_weights || !d_kv || !d_workspace) return fail(DG_ERR_INVALID, "weights, KV cache and workspace are required");
  if (capacity < desc->canvas) return fail(DG_ERR_CAPACITY, "KV capacity must hold at least one canvas");
  if (capacity > (1ll << 30)) return fail(DG_ERR_CAPACITY, "KV capacity too large");
  if (capacity % kVBlock != 0) return fail(DG_ERR_CAPACITY, "KV capacity must be a multiple of 32");
  for (const void* p : {d_weights, d_kv, d_workspace})
    if (reinterpret_cast<uintptr_t>(p) % 256 != 0) return fail(DG_ERR_INVALID, "device buffers must be 256-byte aligned");
  const WsLayout wl = ws_layout(*desc, capacity);
  if (ws_bytes < wl.total) return fail(DG_ERR_CAPACITY, "workspace too small (see dg_workspace_size)");
  DG_TRY(zero_fill(d_workspace, wl.total, nullptr));
  // attention reads whole 32-position V blocks and weights unused positions by 0: keep them finite
  DG_TRY(zero_fill(d_kv, dg_kv_bytes(desc, capacity), nullptr));
  if (desc->rope_theta > 0.f)
    DG_TRY(rope_table(desc->rope_theta, desc->head_dim, capacity,
                      reinterpret_cast<float2*>(static_cast<char*>(d_workspace) + wl.rope), nullptr));
  DG_HIP(hipStreamSynchronize(nullptr));
  dg_ctx* c = new dg_ctx;
  c->d = *desc;
  c->w = static_cast<char*>(d_weights);
  c->kv = static_cast<char*>(d_kv);
  c->cap = capacity;
  c->len = 0;
  c->ws = static_cast<char*>(d_workspace);
  c->ws_bytes = ws_bytes;
  c->wl = weight_layout(*desc);
  c->wsl = wl;
  if (hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking) != hipSuccess ||
      hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess ||
      hipHostMalloc(reinterpret_cast<void**>(&c->stop_host), sizeof(dg_stop_state) * dg_ctx::kStopSlots,
                    hipHostMallocDefault) != hipSuccess) {
    dg_ctx_destroy(c);
    return fail(DG_ERR_HIP, "could not create the context's streams, events and pinned stop slots");
  }
  for (hipEvent_t& e : c->stop_ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      dg_ctx_destroy(c);
      return fail(DG_ERR_HIP, "could not create the stop read-back events");
    }
  *out = c;
  return DG_OK;
}

int dg_ctx_destroy(dg_ctx* ctx) {
  if (ctx) {
    (void)hipDeviceSynchronize();
    for (StepGraph& g : ctx->graphs) drop_graph(g);
    if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
    if (ctx->aux) (void)hipStreamSynchronize(ctx->aux);
    if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
    if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
    if (ctx->aux) (void)hipStreamDestroy(ctx->aux);
    for (hipEvent_t e : ctx->stop_ev)
      if (e) (void)hipEventDestroy(e);
    if (ctx->stop_host) (void)hipHostFree(ctx->stop_host);
  }
  delete ctx;
  return DG_OK;
}

int dg_ctx_set_weights(dg_ctx* ctx, void* d_weights) {
  DG_TRY(check_ctx(ctx));
  if (!d_weights) return fail(DG_ERR_INVALID, "d_weights is NULL");
  if (reinterpret_cast<uintptr_t>(d_weights) % 256 != 0)
    return fail(DG_ERR_INVALID, "device buffers must be 256-byte aligned");
  DG_HIP(hipDeviceSynchronize());
  for (StepGraph& g : ctx->graphs) drop_graph(g);
  ctx->w = static_cast<char*>(d_weights);
  return DG_OK;
}

int dg_ctx_use_graphs(dg_ctx* ctx, int32_t on) {
  DG_TRY(check_ctx(ctx));
  ctx->use_graphs = on != 0;
  if (!ctx->use_graphs) {
    DG_HIP(hipDeviceSynchronize());
    for (StepGraph& g : ctx->graphs) drop_graph(g);
  }
  return DG_OK;
}

int dg_ctx_use_expert_fp8(dg_ctx* ctx, const void* d_fp8) {
  DG_TRY(check_ctx(ctx));
  if (d_fp8) {
    DG_TRY(check_fp8_desc(&ctx->d));
    if (reinterpret_cast<uintptr_t>(d_fp8) % 256 != 0) return fail(DG_ERR_INVALID, "d_fp8 must be 256-byte aligned");
  }
  DG_HIP(hipDeviceSynchronize());
  for (StepGraph& g : ctx->graphs) drop_graph(g);
  ctx->fp8 = static_cast<const char*>(d_fp8);
  if (d_fp8) ctx->fl = fp8_layout(ctx->d);
  return DG_OK;
}

int dg_ctx_fuse_sampler_stats(dg_ctx* ctx, const dg_sched* sched) {
  DG_TRY(check_ctx(ctx));
  if (sched) {
    DG_TRY(check_sched(sched, 0));
    if (ctx->d.dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "sampler records in the LM head: bf16 models only");
    if (sched->mode & DG_SCHED_SAMPLE)
      return fail(DG_ERR_UNSUPPORTED, "categorical sampling perturbs every logit: it needs the sampler's own pass");
  }
  DG_HIP(hipDeviceSynchronize());
  for (StepGraph& g : ctx->graphs) drop_graph(g);  // the captured LM head launch changes
  ctx->fuse_stats = sched != nullptr;
  if (sched) ctx->fuse_sched = *sched;
  return DG_OK;
}

int dg_sample_canvas_fused(dg_ctx* ctx, const dg_sched* sched, int32_t step, int32_t block, int32_t* d_canvas,
                           int32_t* d_pred, uint8_t* d_accept, float* d_entropy, float* d_row_stats,
                           dg_stop_state* d_stop, void* d_workspace, size_t ws_bytes, void* stream) {
  DG_TRY(check_ctx(ctx));
  DG_TRY(check_sched(sched, step));
  if (!ctx->fuse_stats) return fail(DG_ERR_INVALID, "the LM head does not produce sampler records (dg_ctx_fuse_sampler_stats)");
  if (!same_temperatures(ctx->fuse_sched, *sched))
    return fail(DG_ERR_INVALID, "the schedule's temperatures differ from the LM head's sampler records");
  if (sched->mode & DG_SCHED_SAMPLE)
    return fail(DG_ERR_UNSUPPORTED, "categorical sampling perturbs every logit: it needs the sampler's own pass");
  if (!d_canvas || !d_pred || !d_stop || !d_workspace)
    return fail(DG_ERR_INVALID, "d_canvas, d_pred, d_stop and d_workspace are required");
  if (block < 0) return fail(DG_ERR_INVALID, "block must be >= 0");
  const int C = ctx->d.canvas;
  if (ws_bytes < sample_workspace_bytes(C, ctx->d.vocab) || reinterpret_cast<uintptr_t>(d_workspace) % 256 != 0)
    return fail(DG_ERR_INVALID, "d_workspace must be 256-aligned and hold dg_sample_workspace_size(canvas, vocab) bytes");
  return launch_sample_from_block_recs(wsp<void>(ctx, ctx->wsl.vrecs), vocab_blocks(ctx->d.vocab), C, ctx->d.vocab,
                                       temperature(*sched, step), *sched, step, block, d_canvas, d_pred, d_accept,
                                       d_entropy, d_row_stats, d_stop, d_workspace, as_stream(stream));
}

int64_t dg_kv_length(const dg_ctx* ctx) { return ctx ? ctx->len : -1; }

int64_t dg_ctx_graph_captures(const dg_ctx* ctx) { return ctx ? ctx->captures : -1; }

int dg_kv_set_length(dg_ctx* ctx, int64_t length) {
  DG_TRY(check_ctx(ctx));
  if (length < 0 || length > ctx->cap) return fail(DG_ERR_CAPACITY, "length outside [0, capacity]");
  // the device copy is written behind everything already queued on any stream
  DG_HIP(hipDeviceSynchronize());
  DG_TRY(store_i32(wsp<int32_t>(ctx, ctx->wsl.len_dev), static_cast<int32_t>(length), nullptr));
  DG_HIP(hipStreamSynchronize(nullptr));
  ctx->len = length;
  return DG_OK;
}

int dg_prefill_kv(dg_ctx* ctx, const int32_t* d_prompt_ids, int32_t n_prompt, void* stream) {
  DG_TRY(check_ctx(ctx));
  if (n_prompt < 0) return fail(DG_ERR_SHAPE, "n_prompt must be >= 0");
  if (n_prompt > 0 && !d_prompt_ids) return fail(DG_ERR_INVALID, "d_prompt_ids is NULL");
  if (ctx->len + n_prompt > ctx->cap) return fail(DG_ERR_CAPACITY, "prompt does not fit in the KV cache");
  return encode(ctx, d_prompt_ids, n_prompt, as_stream(stream));
}

int dg_denoise_step(dg_ctx* ctx, const int32_t* d_canvas, int32_t step, const void* d_prev_logits,
                    const float* d_prev_row_stats, float prev_temperature, void* d_logits, void* stream) {
  DG_TRY(check_ctx(ctx));
  if (!d_canvas || !d_logits) return fail(DG_ERR_INVALID, "d_canvas and d_logits are required");
  if (d_prev_logits && (!d_prev_row_stats || !(prev_temperature > 0.f) || !isfinite(prev_temperature)))
    return fail(DG_ERR_INVALID, "self-conditioning needs row stats and a positive temperature");
  if (ctx->len + ctx->d.canvas > ctx->cap) return fail(DG_ERR_CAPACITY, "no room for the canvas in the KV cache");
  if (ctx->fuse_stats && (step < 0 || step >= ctx->fuse_sched.max_steps))
    return fail(DG_ERR_INVALID, "step outside the schedule the LM head's sampler records follow");
  return denoise(ctx, step, d_canvas, d_prev_logits, d_prev_row_stats, prev_temperature, d_logits, as_stream(stream));
}

int dg_commit_block(dg_ctx* ctx, const int32_t* d_block_ids, void* stream) {
  DG_TRY(check_ctx(ctx));
  if (!d_block_ids) return fail(DG_ERR_INVALID, "d_block_ids is NULL");
  if (ctx->len + ctx->d.canvas > ctx->cap) return fail(DG_ERR_CAPACITY, "block does not fit in the KV cache");
  return encode(ctx, d_block_ids, ctx->d.canvas, as_stream(stream));
}

int dg_forward_layer(dg_ctx* ctx, int32_t layer, float* d_x, int32_t rows, int32_t causal, void* stream) {
  DG_TRY(check_ctx(ctx));
  if (layer < 0 || layer >= ctx->d.n_layers) return fail(DG_ERR_INVALID, "layer out of range");
  if (!d_x) return fail(DG_ERR_INVALID, "d_x is NULL");
  if (rows < 1 || rows > pass_rows(ctx->d)) return fail(DG_ERR_SHAPE, "rows must be in [1, max(canvas, prefill_rows)]");
  if (ctx->len + rows > ctx->cap) return fail(DG_ERR_CAPACITY, "rows do not fit in the KV cache");
  hipStream_t s = as_stream(stream);
  DG_TRY(rmsnorm(d_x, wsp<void>(ctx, ctx->wsl.h), rows, ctx->d.d_model, ctx->d.rms_eps, ctx->d.dtype, s));
  return layer_forward(ctx, layer, d_x, rows, static_cast<int>(ctx->len), nullptr, causal != 0, false, s);
}

int dg_generate_block(dg_ctx* ctx, const dg_sched* sched, int32_t block, void* d_logits, int32_t* d_block_out,
                      int32_t commit, int32_t* steps_out, void* stream) {
  DG_TRY(check_ctx(ctx));
  DG_TRY(check_sched(sched, 0));
  if (!d_logits || !d_block_out) return fail(DG_ERR_INVALID, "d_logits and d_block_out are required");
  if (block < 0) return fail(DG_ERR_INVALID, "block must be >= 0");
  const int need = ctx->d.canvas * (commit ? 1 : 0);
  if (ctx->len + ctx->d.canvas > ctx->cap || ctx->len + need > ctx->cap)
    return fail(DG_ERR_CAPACITY, "no room for the canvas in the KV cache");
  hipStream_t s = as_stream(stream);
  const WsLayout& w = ctx->wsl;
  const int C = ctx->d.canvas;
  int32_t* canvas = wsp<int32_t>(ctx, w.canvas);
  int32_t* pred = wsp<int32_t>(ctx, w.pred);
  float* stats = wsp<float>(ctx, w.row_stats);
  dg_stop_state* stop = wsp<dg_stop_state>(ctx, w.stop);
  DG_TRY(launch_init_canvas(sched->seed, block, C, ctx->d.vocab, canvas, stop, s));
  // Each step's stop state is copied to a pinned slot behind the step. The host reads a step's copy
  // only when that step could have stopped: under the two-fold rule the stable count starts at 0 on
  // step 0 and grows by at most one a step, so a step whose count cannot have reached stable_needed
  // cannot stop, and the next step is launched without waiting for it (the device never idles
  // between such steps). With the either-condition rule every step could stop and is read.
  // the LM head's records serve this schedule when they follow its temperatures
  const bool fused = ctx->fuse_stats && same_temperatures(ctx->fuse_sched, *sched);
  if (ctx->fuse_stats && !fused)
    return fail(DG_ERR_INVALID, "the schedule's temperatures differ from the LM head's sampler records");
  const bool either = (sched->mode & DG_SCHED_STOP_EITHER) != 0;
  int known = -1, c_known = 0;  // the last step read, and its stable count
  auto could_stop = [&](int j) {
    const int cap = known < 0 ? j : c_known + (j - known);  // most the stable count can be at step j
    return either || cap >= sched->stable_needed;
  };
  int enq = 0, steps = 0;
  bool stopped = false;
  float prev_t = 0.f;
  while (!stopped) {
    // the earliest unread step that could have stopped must be read before another step starts;
    // so must the oldest one when every slot holds an unread step
    int j = known + 1;
    while (j < enq && !could_stop(j)) ++j;
    if (j == enq && enq - known > dg_ctx::kStopSlots - 1) j = known + 1;
    if (j < enq) {
      DG_HIP(hipEventSynchronize(ctx->stop_ev[j % dg_ctx::kStopSlots]));
      const dg_stop_state& st = ctx->stop_host[j % dg_ctx::kStopSlots];
      known = j;
      c_known = st.stable_count;
      if (st.stopped) {
        stopped = true;
        steps = j + 1;
      }
      continue;
    }
    if (enq == sched->max_steps) break;
    const int step = enq;
    const float T = temperature(*sched, step);
    DG_TRY(denoise(ctx, step, canvas, step > 0 ? d_logits : nullptr, stats, prev_t, d_logits, s));
    if (fused)
      DG_TRY(launch_sample_from_block_recs(wsp<void>(ctx, w.vrecs), vocab_blocks(ctx->d.vocab), C, ctx->d.vocab, T,
                                           *sched, step, block, canvas, pred, wsp<uint8_t>(ctx, w.accept),
                                           wsp<float>(ctx, w.entropy), stats, stop, wsp<void>(ctx, w.samp), s));
    else
      DG_TRY(launch_sample(d_logits, ctx->d.dtype, C, ctx->d.vocab, T, *sched, step, block, canvas, pred,
                           wsp<uint8_t>(ctx, w.accept), wsp<float>(ctx, w.entropy), stats, stop,
                           wsp<void>(ctx, w.samp), s));
    DG_HIP(hipMemcpyAsync(&ctx->stop_host[step % dg_ctx::kStopSlots], stop, sizeof(dg_stop_state),
                          hipMemcpyDeviceToHost, s));
    DG_HIP(hipEventRecord(ctx->stop_ev[step % dg_ctx::kStopSlots], s));
    prev_t = T;
    ++enq;
  }
  if (!stopped) steps = enq;  // max_steps ran; none of them stopped
  DG_HIP(hipMemcpyAsync(d_block_out, pred, C * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  if (steps_out) *steps_out = steps;
  if (commit) DG_TRY(encode(ctx, d_block_out, C, s));
  return DG_OK;
}

int dg_ctx_buffer(const dg_ctx* ctx, int32_t which, void** d_ptr, size_t* bytes) {
  if (!ctx || !d_ptr) return fail(DG_ERR_INVALID, "ctx and d_ptr are required");
  const dg_model_desc& d = ctx->d;
  const WsLayout& w = ctx->wsl;
  const size_t C = d.canvas, es = esize(d);
  const size_t K = d.top_k, sel_l = static_cast<size_t>(ctx->last_layer) * w.sel_layer * 4;
  size_t off, n;
  switch (which) {
    case DG_BUF_X: off = w.x; n = C * d.d_model * 4; break;
    case DG_BUF_H: off = w.h; n = C * d.d_model * es; break;
    case DG_BUF_ROUTER_LOGITS: off = w.rlog; n = C * d.n_experts * 4; break;
    case DG_BUF_SEL: off = w.sel + sel_l; n = C * K * 4; break;
    case DG_BUF_GATE: off = w.gate + sel_l; n = C * K * 4; break;
    case DG_BUF_SEL_LAYERS: off = w.sel; n = static_cast<size_t>(d.n_layers) * w.sel_layer * 4; break;
    case DG_BUF_SC: off = w.sc; n = C * d.d_model * 4; break;
    case DG_BUF_CANVAS: off = w.canvas; n = C * 4; break;
    case DG_BUF_PRED: off = w.pred; n = C * 4; break;
    case DG_BUF_STOP: off = w.stop; n = sizeof(dg_stop_state); break;
    case DG_BUF_ENTROPY: off = w.entropy; n = C * 4; break;
    case DG_BUF_ROW_STATS: off = w.row_stats; n = C * 8; break;
    case DG_BUF_ACCEPT: off = w.accept; n = C; break;
    case DG_BUF_Q: off = w.q; n = C * d.n_q_heads * d.head_dim * es; break;
    case DG_BUF_ATTN: off = w.o; n = C * d.n_q_heads * d.head_dim * es; break;
    case DG_BUF_SHARED_ACT: off = w.sh_act; n = C * d.d_shared * es; break;
    case DG_BUF_SLOT_OUT: off = w.slot_out; n = C * d.top_k * d.d_model * 4; break;
    case DG_BUF_SLOT_OF: off = w.slot_of; n = C * d.top_k * 4; break;
    case DG_BUF_OFFSETS: off = w.offsets; n = (2 * static_cast<size_t>(d.n_experts) + 1) * 4; break;
    default: return fail(DG_ERR_INVALID, "unknown buffer");
  }
  *d_ptr = ctx->ws + off;
  if (bytes) *bytes = n;
  return DG_OK;
}

}  // extern "C"
