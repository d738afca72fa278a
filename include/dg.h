/*
 * dg.h - C ABI of libdg, a uniform-state discrete-diffusion ("canvas
 * denoising") step for AMD Instinct MI355X (gfx950).
 *
 * Method sources, cited by page title and section:
 *  [P1] molayo1419.me, "Running the diffusion LLM DiffusionGemma on Modal and
 *       visualising the denoising steps in a browser".
 *  [P2] axbrief.com, "DiffusionGemma: Google's 26B MoE model that generates
 *       text like images".
 *  [P3] juhoplayground.github.io, "DiffusionGemma - parallel text generation
 *       and diffusion-based language models".
 *  [P4] marrrang.tistory.com, "[AI] DiffusionGemma deep dive - Uniform State
 *       Diffusion and inference architecture".
 *
 * Conventions for every call:
 *  - Pointers named d_* are device pointers (HIP global memory) owned by the
 *    caller; the library never frees them. Pointers without the prefix are
 *    host pointers read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; the call returns before the GPU
 *    is done unless stated otherwise.
 *  - Return value: DG_OK (0) or a negative DG_ERR_* code. Argument, shape and
 *    capacity checks happen before anything is enqueued, so a failing call has
 *    no side effect. A HIP launch failure returns DG_ERR_HIP. dg_last_error()
 *    gives a message for the last failing call on the calling thread.
 *  - Matrices are row-major. Model weights are stored [out_features,
 *    in_features]. dtype DG_BF16 means bf16 weights, KV cache, logits and
 *    GEMM operands with fp32 accumulation and an fp32 residual stream;
 *    DG_F32 means fp32 everywhere.
 *  - Calls that share a context or a workspace must not overlap in time
 *    (serialise them on one stream).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DG_OK = 0,
  DG_ERR_INVALID = -1,     /* null pointer or out-of-range argument */
  DG_ERR_SHAPE = -2,       /* inconsistent sizes */
  DG_ERR_CAPACITY = -3,    /* KV cache capacity or workspace too small */
  DG_ERR_UNSUPPORTED = -4, /* valid but not implemented (e.g. head_dim) */
  DG_ERR_HIP = -5          /* HIP runtime error */
};

enum { DG_BF16 = 0, DG_F32 = 1 };

/* Model shape. The pages fix canvas = 256 and 8 of 128 experts + 1 shared
 * ([P4] "Gemma-based MoE backbone", table); the rest is the caller's. */
typedef struct dg_model_desc {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_q_heads;
  int32_t n_kv_heads;   /* n_q_heads must be a multiple of n_kv_heads */
  int32_t head_dim;     /* 64 or 128 */
  int32_t n_experts;
  int32_t top_k;
  int32_t d_expert;     /* hidden width of one routed expert */
  int32_t d_shared;     /* hidden width of the shared expert */
  int32_t gated;        /* 1: GeLU(h Wg) * (h Wu); 0: GeLU(h Wu) */
  int32_t vocab;        /* tied embedding / LM head rows */
  int32_t canvas;       /* canvas positions per denoising step (<= 256) */
  int32_t d_selfcond;   /* hidden width of the self-conditioning FFN */
  int32_t dtype;        /* DG_BF16 or DG_F32 */
  float rms_eps;
  int32_t renorm_gates; /* 0: gate = softmax prob of the expert (default) */
} dg_model_desc;

/* Sampler settings ([P4] "Standard sampling settings" table: 48 steps,
 * temperature 0.8 -> 0.4 linear, entropy bound 0.1, stop threshold 0.005;
 * [P4] "Two-Fold Adaptive Stopping": two consecutive equal predictions). */
typedef struct dg_sched {
  int32_t max_steps;
  float t_start;
  float t_end;
  float entropy_bound;      /* accept a position iff its entropy <= bound */
  float stop_mean_entropy;  /* stop needs canvas mean entropy < this ... */
  int32_t stable_needed;    /* ... and this many consecutive equal predictions */
  uint64_t seed;            /* Philox key */
} dg_sched;

/* Device-resident stop state, 16 bytes, updated by dg_sample_canvas. */
typedef struct dg_stop_state {
  float mean_entropy;   /* canvas mean entropy of the last sampled step */
  int32_t stable_count; /* consecutive steps whose argmax equalled the previous */
  int32_t stopped;      /* 1 once the two-fold stop fired */
  int32_t steps_run;    /* steps sampled so far for this canvas */
} dg_stop_state;

typedef struct dg_ctx dg_ctx;

/* ---------------------------------------------------------------- misc */
const char* dg_last_error(void);
const char* dg_version(void);

/* Temperature of step `step`: t_start + (t_end - t_start) * step / (max_steps - 1),
 * evaluated in double and rounded once to float ([P4] "Standard sampling
 * settings": linear decay; [P3] "Inference mechanism": logits scheduler).
 * Returns NaN for a null sched. */
float dg_temperature(const dg_sched* sched, int32_t step);

/* Per-kernel timing (tracing). dg_profile_enable(1, n) creates a pool of
 * HIP events for up to n kernel launches; while enabled, every libdg kernel
 * launch records an event pair on its stream. dg_profile_enable(0, 0) turns
 * it off and frees the pool. dg_profile_report waits for the recorded events
 * and writes a JSON object {kernel: {count, total_us, avg_us}} into buf
 * (host, cap bytes), then clears the record. Not for use during graph
 * capture. */
int dg_profile_enable(int32_t on, int32_t max_launches);
int dg_profile_report(char* buf, size_t cap);

/* ------------------------------------------------------------- sampler */

/* Bytes of device scratch dg_sample_canvas needs for rows x vocab logits. */
size_t dg_sample_workspace_size(int32_t rows, int32_t vocab);

/* Canvas initialisation: d_canvas[i] = token(Philox4x32-10(key = seed,
 * counter = (i, 0, block, 0)) word 0), token(r) = floor(r * vocab / 2^32)
 * ([P3] "Inference mechanism": the sampler starts from uniformly random
 * tokens; [P4] "Reverse diffusion process", step 1). Also resets *d_stop to
 * {mean_entropy = +inf, stable_count = 0, stopped = 0, steps_run = 0}.
 * d_canvas: int32[canvas]. d_stop may be NULL. */
int dg_init_canvas(const dg_sched* sched, int32_t block, int32_t canvas, int32_t vocab,
                   int32_t* d_canvas, dg_stop_state* d_stop, void* stream);

/* One entropy-bounded sampling step over logits [rows x vocab]
 * ([P3] "Inference mechanism": entropy-bounded sampler; [P4] "Standard
 * sampling settings"; [P4] "Two-Fold Adaptive Stopping"). With
 * T = dg_temperature(sched, step), per row i:
 *   p = softmax(l_i / T); H_i = -sum p ln p (nats);
 *   pred_i = argmax l_i (lowest index on ties);
 *   accept_i = H_i <= entropy_bound;
 *   canvas_i = accept_i ? pred_i : token(Philox(seed; i, step, block, 1) word 0);
 *   row_stats_i = (max_v l_iv, ln sum_v exp((l_iv - max) / T)).
 * Over the canvas: mean_entropy = mean H; stable_count = (step > 0 and
 * pred == previous pred) ? stable_count + 1 : 0; stopped = mean_entropy <
 * stop_mean_entropy and stable_count >= stable_needed; steps_run = step + 1.
 * If d_stop->stopped is already 1 the call changes nothing (so a whole step
 * budget can be enqueued without reading the state back).
 *  d_logits    [rows x vocab] bf16 or fp32 (dtype), read once.
 *  d_canvas    int32[rows], written (next canvas).
 *  d_pred      int32[rows], in: previous step's argmax; out: this step's.
 *  d_accept    uint8[rows], d_entropy float[rows], d_row_stats float[rows x 2]
 *              (any of these three may be NULL).
 *  d_workspace >= dg_sample_workspace_size(rows, vocab) bytes, 256-aligned.
 * rows in [1, 65535], vocab in [1, 2^31 - 1]. */
int dg_sample_canvas(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab,
                     const dg_sched* sched, int32_t step, int32_t block,
                     int32_t* d_canvas, int32_t* d_pred, uint8_t* d_accept, float* d_entropy,
                     float* d_row_stats, dg_stop_state* d_stop,
                     void* d_workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------- synthetic inputs */
/* Seeded synthetic data (no method arithmetic): value i of stream (seed, tid)
 * is the Irwin-Hall sum of the four 16-bit fields of a SplitMix64-based hash,
 * scaled to standard deviation sigma by one float multiply, then rounded to
 * bf16 (nearest-even) when dtype is DG_BF16. Bit-identical to the host
 * generator the tests use. */
int dg_synth_normal(uint64_t seed, uint64_t tid, int64_t n, float sigma, int32_t dtype,
                    void* d_out, void* stream);
/* Uniform ids in [0, vocab). */
int dg_synth_uniform_ids(uint64_t seed, uint64_t tid, int64_t n, int32_t vocab,
                         int32_t* d_out, void* stream);
/* bf16 logits [rows x vocab]: background sigma, +peak added at one uniform
 * column in about 70% of the rows (buffer index `step` selects the stream). */
int dg_synth_planted_logits(uint64_t seed, int32_t step, int32_t rows, int32_t vocab,
                            float sigma, float peak, void* d_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
