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
  float rope_theta;     /* 0: no positional encoding (default); > 0: rotary
                         * embedding of queries and keys at their cache
                         * positions p, pairs (j, j + head_dim/2) turned by
                         * p * rope_theta^(-2j/head_dim) (the Gemma family's
                         * form; [P3] "Encoder-denoiser design" names the
                         * backbone, the pages give no positional scheme) */
  int32_t prefill_rows; /* 0: prefill and commit run in chunks of `canvas`
                         * rows; else chunk rows in [canvas, 4096] (more
                         * than 256 needs n_experts <= 128): the workspace
                         * grows with it, and chunks of more than 256 rows
                         * run the routed experts (bf16) as token-tiled
                         * GEMMs of 128 tokens per workgroup */
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
  int32_t mode;             /* 0, or DG_SCHED_* flags: the sampler variants below */
  int32_t reserved;         /* 0 */
} dg_sched;

/* Sampler variants ([P3] "Inference mechanism"), flags of dg_sched.mode:
 * DG_SCHED_STOP_EITHER: the canvas stops when either condition holds (mean
 *   entropy below the threshold, or stable_needed consecutive equal
 *   predictions) instead of both;
 * DG_SCHED_ACCEPT_GROUP: the accepted positions are a group: taken in
 *   increasing entropy (lower position first on ties), the longest run whose
 *   running entropy total (float, in that order) stays <= entropy_bound;
 * DG_SCHED_SAMPLE: ([P4] "Standard sampling settings": the temperature
 *   explores early) an accepted position keeps a token drawn from
 *   softmax(l / T) by Gumbel-max, argmax_v l_v / T - ln(-ln u_v), instead of
 *   the argmax; u_v = (r >> 8 + 1/2) / 2^24 with r = output word v % 4 of
 *   Philox(seed; i, step, block, 2 + 4 (v / 4)). pred (the stop rule's
 *   predictions) stays the argmax. Needs vocab % 8 == 0. */
enum { DG_SCHED_STOP_EITHER = 1, DG_SCHED_ACCEPT_GROUP = 2, DG_SCHED_SAMPLE = 4 };

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
 * capture. dg_profile_only(name) restricts recording to the launch sites of
 * that name (as the report keys them; NULL: all), so a timed region can carry
 * the events of one kernel only. */
int dg_profile_enable(int32_t on, int32_t max_launches);
int dg_profile_only(const char* name);
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
 *  d_workspace >= dg_sample_workspace_size(rows, vocab) bytes, 256-aligned
 *              (per-chunk partial records); calls sharing it must not overlap.
 * Two kernels: a split-row partial pass and a one-workgroup finalize.
 * rows in [1, 65535], vocab in [1, 2^31 - 1]. */
int dg_sample_canvas(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab,
                     const dg_sched* sched, int32_t step, int32_t block,
                     int32_t* d_canvas, int32_t* d_pred, uint8_t* d_accept, float* d_entropy,
                     float* d_row_stats, dg_stop_state* d_stop,
                     void* d_workspace, size_t ws_bytes, void* stream);

/* dg_sample_canvas without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the per-chunk partial records live in a
 * static device array of the library, 1 MiB per device (held until the process
 * ends), whose address is looked up once per device on the first call there.
 * Same arguments, results and limits as dg_sample_canvas otherwise; calls whose
 * dg_sample_workspace_size(rows, vocab) exceeds 1 MiB fail with
 * DG_ERR_CAPACITY before anything is enqueued (a canvas of up to 256 rows needs
 * at most 96 KiB at any vocabulary). Nothing is
 * allocated; every call on one device shares its array, so calls that overlap
 * in time on one device race (serialise them on one stream). */
int dg_sample_canvas_static(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab,
                            const dg_sched* sched, int32_t step, int32_t block, int32_t* d_canvas,
                            int32_t* d_pred, uint8_t* d_accept, float* d_entropy, float* d_row_stats,
                            dg_stop_state* d_stop, void* stream);

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
/* bf16 logits [rows x vocab]: background of standard deviation sigma (the
 * sum of twelve 16-bit hash fields, three hashes per value: tails to 6 sigma),
 * +peak added at one uniform column in about 70% of the rows (buffer index
 * `step` selects the stream). */
int dg_synth_planted_logits(uint64_t seed, int32_t step, int32_t rows, int32_t vocab,
                            float sigma, float peak, void* d_out, void* stream);
/* Fill a packed weight buffer (see dg_weight_tensor) with synthetic values of
 * standard deviation sigma: tensor (kind, layer, expert) uses stream
 * tid = 1 (embedding), 2 / 3 (self-conditioning W1 / W2),
 * 2^20 + 64 layer + {0 q, 1 k, 2 v, 3 o, 4 router, 5 shared gate, 6 shared up,
 * 7 shared down}, 2^32 + 8 (1024 layer + expert) + {0 gate, 1 up, 2 down};
 * element i is the row-major index inside the tensor (routed-expert tensors
 * are then stored fragment-tiled, as dg_load_weight would store them). Then
 * derives the transposed embedding (dg_prepare_weights). */
int dg_synth_fill_weights(const dg_model_desc* desc, uint64_t seed, float sigma, void* d_weights,
                          void* stream);

/* Calibration of memory bandwidth: read `bytes` (a multiple of 16) of d_src
 * once with a plain streaming kernel (`blocks` workgroups of 256 threads,
 * grid-stride nontemporal 16-byte loads) and write one XOR-folded word per
 * workgroup to d_sink (uint32[blocks]). Its duration bounds what a streaming
 * kernel of this library can reach on the device; it computes nothing of the
 * method. */
int dg_stream_read(const void* d_src, int64_t bytes, uint32_t* d_sink, int32_t blocks, void* stream);

/* --------------------------------------------------------------- model */
/* Weight tensors inside the packed, caller-owned weight buffer. */
enum {
  DG_W_EMBED = 0,    /* [vocab x d_model], tied input embedding and LM head */
  DG_W_EMBED_T = 1,  /* [d_model x vocab], derived copy of EMBED transposed, stored tiled */
  DG_W_SC1 = 2,      /* [d_selfcond x d_model] self-conditioning FFN, first */
  DG_W_SC2 = 3,      /* [d_model x d_selfcond] self-conditioning FFN, second */
  DG_W_Q = 4,        /* [n_q_heads*head_dim x d_model] (per layer) */
  DG_W_K = 5,        /* [n_kv_heads*head_dim x d_model] */
  DG_W_V = 6,        /* [n_kv_heads*head_dim x d_model] */
  DG_W_O = 7,        /* [d_model x n_q_heads*head_dim] */
  DG_W_ROUTER = 8,   /* [n_experts x d_model] */
  DG_W_SH_GATE = 9,  /* [d_shared x d_model] (gated models only) */
  DG_W_SH_UP = 10,   /* [d_shared x d_model] */
  DG_W_SH_DOWN = 11, /* [d_model x d_shared] */
  DG_W_EX_GATE = 12, /* [d_expert x d_model] (per layer and expert; gated only) */
  DG_W_EX_UP = 13,   /* [d_expert x d_model] */
  DG_W_EX_DOWN = 14  /* [d_model x d_expert] */
};

/* Total bytes of the packed weight buffer (every tensor 256-byte aligned). */
size_t dg_weights_bytes(const dg_model_desc* desc);
/* Byte offset and logical [rows x cols] shape of one tensor; layer / expert
 * are ignored where they do not apply. Q, K and V of a layer are adjacent
 * (one fused projection), as are gate and up of the shared expert. Every
 * tensor except the embedding and the routed experts' is stored row-major at
 * that offset. DG_W_EMBED and the routed experts' matrices (DG_W_EX_*) are
 * stored fragment-tiled so the LM head and expert kernels stream contiguous
 * memory: 16-row x 32-column tiles of 512 elements in which element 8 l + j
 * is row l % 16, column 8 (l / 16) + j; embedding: tiles ordered [32-row
 * group][column tile][the group's 2 16-row blocks]; gate/up: tiles ordered [32-feature group][column tile][gate rows 0-15,
 * gate rows 16-31, up rows 0-15, up rows 16-31 of the group] (up alone when
 * ungated), down: [64-row group][column tile][the group's 4 16-row
 * blocks]. DG_W_EMBED_T, the [d_model x vocab] operand of the
 * self-conditioning product, is tiled like the embedding: [32-row group of
 * d_model][vocabulary tile of 32][the group's 2 16-row blocks]. For
 * DG_W_EX_GATE / DG_W_EX_UP the offset is the start of the expert's shared
 * gate/up region. Write them with dg_load_weight. */
int dg_weight_tensor(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert,
                     size_t* offset, int64_t* rows, int64_t* cols);
/* Store one tensor from a row-major [rows x cols] device array d_src of the
 * model dtype (shape as dg_weight_tensor reports) into the weight buffer,
 * tiling the routed-expert kinds; asynchronous on `stream`; d_src must stay
 * valid until the copy has run. DG_W_EMBED_T is rejected (derived by
 * dg_prepare_weights). Errors: DG_ERR_INVALID for bad kind / layer / expert
 * or NULL pointers. */
int dg_load_weight(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert,
                   const void* d_src, void* d_weights, void* stream);
/* Rebuild DG_W_EMBED_T from DG_W_EMBED (call after loading weights). */
int dg_prepare_weights(const dg_model_desc* desc, void* d_weights, void* stream);

/* FP8 routed experts (opt-in; [P2] "24GB GPU: practical adoption and
 * running conditions" lists quantised GGUF builds of the model, the 8-bit
 * one at about half the bf16 footprint, and [P1] "Summary" points local runs
 * at them; the format here is this library's own 8-bit storage): a
 * separate caller-owned device buffer holding every layer's routed-expert
 * matrices as OCP E4M3 codes (bias 7, 3 fraction bits, subnormals in units
 * of 2^-9, no infinities, largest finite 448) with one float32 scale per
 * output row (a gate / up feature, a down output): s = max|w| / 448 (1 for
 * an all-zero row), code = E4M3(w / s) rounded to nearest-even and saturated
 * at +-448, both divisions the correctly rounded float32 ones; the model
 * then computes with code * s. The bf16 weights stay in use for everything
 * else. bf16 models with d_expert and d_model multiples of 64 only. */
/* Bytes of the FP8 expert buffer (0 for an invalid or unsupported desc). Per
 * layer, 256-byte aligned: gate/up codes [expert][gw * d_expert * d_model]
 * (gw = 2 gated, 1 not), down codes [expert][d_model * d_expert], gate/up
 * scales float32 [expert][gw][d_expert], down scales [expert][d_model]. The
 * codes follow the routed experts' tile order (dg_weight_tensor) at one byte
 * per element, with k-tiles paired: for column tiles 2p and 2p + 1 of one
 * 16-row block, a 1024-byte block holds at bytes 16 l .. 16 l + 15 element
 * slot l's 8 codes of tile 2p, then its 8 codes of tile 2p + 1 (slot l is row
 * l % 16, columns 8 (l / 16) .. +7 of the tile); blocks ordered [row group]
 * [column pair][the group's row blocks, gate before up]. */
size_t dg_expert_fp8_bytes(const dg_model_desc* desc);
/* Byte offsets inside the FP8 buffer of one routed-expert matrix: the
 * expert's code region (for DG_W_EX_GATE / DG_W_EX_UP the shared gate/up
 * region) and the first float32 scale of that matrix. Errors:
 * DG_ERR_INVALID (bad kind / layer / expert, NULL outputs),
 * DG_ERR_UNSUPPORTED (desc without FP8 support). */
int dg_expert_fp8_tensor(const dg_model_desc* desc, int32_t kind, int32_t layer, int32_t expert,
                         size_t* code_offset, size_t* scale_offset);
/* Quantize every routed expert of the weight buffer into d_fp8
 * (dg_expert_fp8_bytes, 256-byte aligned, caller-owned), asynchronously on
 * `stream`; d_weights is only read. Deterministic: codes and scales depend on
 * the weights alone. Errors: DG_ERR_INVALID (NULL / misaligned buffers),
 * DG_ERR_UNSUPPORTED (fp32 model or widths not multiples of 64). */
int dg_quantize_experts_fp8(const dg_model_desc* desc, const void* d_weights, void* d_fp8, void* stream);

/* KV cache, in the model dtype: keys [n_layers][n_kv_heads][capacity][head_dim]
 * (row-major), then values [n_layers][n_kv_heads][capacity / 32][head_dim][32]:
 * V transposed in blocks of 32 positions, where inside a block slot 8 g + j
 * (g = 0..3) holds position 4 g + j for j < 4 and 16 + 4 g + (j - 4) for
 * j >= 4. capacity must be a multiple of 32. The size includes a tail after
 * the values of (the attention kernel's largest key stage - 32) head_dim-wide
 * positions, 128 - 32 = 96 in this build: attention copies whole stages of V
 * blocks, so the last stage of a key range may read up to that many positions
 * past the capacity (never written, always weighted by zero). */
size_t dg_kv_bytes(const dg_model_desc* desc, int64_t capacity);
/* Scratch the context needs: activations of one layer pass (a canvas, or a
 * prompt / commit chunk of up to max(canvas, prefill_rows) rows), MoE routing
 * tables, the rotary table (capacity positions, when rope_theta > 0), split-K partials,
 * self-conditioning buffers and the sampler state of dg_generate_block. */
size_t dg_workspace_size(const dg_model_desc* desc, int64_t capacity);

/* Create a context over caller-owned weights, KV cache and workspace (none is
 * copied; all must outlive the context). Zero-fills the workspace and the KV
 * cache, fills the rotary table when rope_theta > 0 (blocking, on the default
 * stream) and creates two streams, events and 256 bytes of pinned host
 * memory of its own (default priority). capacity = KV positions, a multiple
 * of 32. The committed length starts at 0. Limits: canvas <= 256, head_dim
 * 64 or 128 (bf16), d_model, head dims, FFN widths and vocab multiples of
 * 64, n_experts <= 256, top_k <= 16. */
int dg_ctx_create(const dg_model_desc* desc, void* d_weights, void* d_kv, int64_t capacity,
                  void* d_workspace, size_t ws_bytes, dg_ctx** out);
/* Waits for the device, then frees the context's own streams, events, pinned
 * host slots and graphs (never the caller's buffers). */
int dg_ctx_destroy(dg_ctx* ctx);
/* Graph replay of the denoising step (default on): the launches of a step are
 * captured into a HIP graph once per (d_canvas, d_logits, d_prev_logits,
 * d_prev_row_stats) pointer set, one graph with self-conditioning and one
 * without, and replayed; a change of those pointers re-captures. The committed
 * KV length and the self-conditioning temperature are read on the device, so
 * commits, prefills and the temperature schedule replay the same graph (a
 * one-thread kernel writes each new value on the stream). Off (0): every
 * launch is issued directly. Steps also run directly while dg_profile_enable
 * is on. */
int dg_ctx_use_graphs(dg_ctx* ctx, int32_t on);
/* Point the context at another copy of its weights ([P3] "Encoder-denoiser
 * design": the denoiser's parameters; [P4] "Gemma-based MoE backbone"):
 * d_weights holds the same dg_weights_bytes bytes in the same layout (a
 * device-to-device copy of the current buffer, or a buffer filled the same
 * way), 256-byte aligned, caller-owned, and must outlive its use. Waits for
 * the device and drops the captured step graphs (the next step re-captures);
 * the KV cache, workspace and every other setting are kept. The old buffer
 * is no longer read once this returns. Errors: DG_ERR_INVALID for NULL or a
 * misaligned pointer. Use: the streaming speed of a weight buffer depends on
 * where its allocation lies in device memory and stays with the allocation,
 * so a caller may time a few copies and keep the fastest. */
int dg_ctx_set_weights(dg_ctx* ctx, void* d_weights);
/* Compute the routed experts from a filled FP8 expert buffer (see
 * dg_quantize_experts_fp8; it must outlive its use and stay unmodified while
 * steps run) in every later prefill, step and commit; NULL returns to the
 * model-dtype weights. Waits for the device and drops captured graphs.
 * Errors: DG_ERR_INVALID (misaligned), DG_ERR_UNSUPPORTED (model without
 * FP8 support). */
int dg_ctx_use_expert_fp8(dg_ctx* ctx, const void* d_fp8);
/* The LM head and the sampler's statistics in one pass ([P3] "Encoder-denoiser
 * design": logits at every canvas position; [P3] "Inference mechanism" and [P4]
 * "Standard sampling settings": the entropy-bounded sampler over them). With a
 * schedule, every later dg_denoise_step(step) also folds its logits, as
 * stored (bf16), into the sampler's split-row records (max, sum 2^u, sum u
 * 2^u, first argmax; u = (l - max) log2(e) / T) at T = the schedule's
 * temperature of that step, one record per row and 256-token vocabulary block;
 * dg_sample_canvas_fused and dg_generate_block then sample from those records
 * instead of reading the logits again (the logits are still written: the next
 * step's self-conditioning reads them). NULL turns this off. Waits for the
 * device and drops captured graphs. Errors: DG_ERR_UNSUPPORTED (an fp32 model,
 * or categorical sampling, whose scores perturb every logit); DG_ERR_INVALID
 * (a bad schedule). dg_generate_block with a schedule of other temperatures
 * fails with DG_ERR_INVALID while this is on. */
int dg_ctx_fuse_sampler_stats(dg_ctx* ctx, const dg_sched* sched);
/* dg_sample_canvas from the records the last dg_denoise_step of this context
 * produced (dg_ctx_fuse_sampler_stats): the same outputs, workspace and
 * arguments, without the logits. `sched` must give step `step` the
 * temperature the records were made at (same max_steps, t_start, t_end), else
 * DG_ERR_INVALID; DG_ERR_UNSUPPORTED for categorical sampling. The records of
 * a row are merged in a fixed order, so the results are reproducible; they
 * equal dg_sample_canvas's up to the rounding of the entropies' sums. */
int dg_sample_canvas_fused(dg_ctx* ctx, const dg_sched* sched, int32_t step, int32_t block, int32_t* d_canvas,
                           int32_t* d_pred, uint8_t* d_accept, float* d_entropy, float* d_row_stats,
                           dg_stop_state* d_stop, void* d_workspace, size_t ws_bytes, void* stream);
int64_t dg_kv_length(const dg_ctx* ctx);
/* Number of denoising-step graphs the context has captured so far (-1 for NULL): a replay
 * re-captures only when the caller's pointers change (see dg_ctx_use_graphs). */
int64_t dg_ctx_graph_captures(const dg_ctx* ctx);
/* Declare the first `length` cache positions valid without computing them
 * (for caches filled by the caller). */
int dg_kv_set_length(dg_ctx* ctx, int64_t length);

/* Encoder mode over the prompt ([P3] "Encoder-denoiser design": the query is
 * processed the standard, causal way and its KV cache is shared with the
 * denoiser; [P4] "System architecture": prefill builds the KV cache). Runs the
 * layers causally over d_prompt_ids (int32[n_prompt]) in chunks of `canvas` (or `prefill_rows`)
 * rows appended at the committed length, then length += n_prompt.
 * DG_ERR_CAPACITY (nothing enqueued) if length + n_prompt > capacity. */
int dg_prefill_kv(dg_ctx* ctx, const int32_t* d_prompt_ids, int32_t n_prompt, void* stream);

/* Denoiser mode, one step ([P3] "Encoder-denoiser design": bidirectional
 * attention over the whole canvas, logits at every canvas position; [P3]
 * "Inference mechanism": self-conditioning). With C = canvas:
 *   if d_prev_logits != NULL: p = softmax(prev_logits / prev_temperature)
 *     rebuilt from d_prev_row_stats (dg_sample_canvas output) inside the
 *     u = p E product (p is never stored), sc = GeLU(u W1^T) W2^T; else sc = 0;
 *   x = E[canvas] + sc; every layer: attention of the C rows over cache
 *   positions [0, length) and the C canvas rows (no mask; the canvas K/V go
 *   to cache slots [length, length + C) as scratch), then the MoE FFN;
 *   logits = RMSNorm(x) E^T -> d_logits [C x vocab] (model dtype).
 * d_prev_logits may alias d_logits (it is read before the LM head writes).
 * Needs length + C <= capacity. `step` is informational. */
int dg_denoise_step(dg_ctx* ctx, const int32_t* d_canvas, int32_t step, const void* d_prev_logits,
                    const float* d_prev_row_stats, float prev_temperature, void* d_logits,
                    void* stream);

/* Block commit ([P3] "Inference mechanism": multi-canvas sampling appends the
 * finished 256 tokens to the prompt and reuses the encoder KV cache; [P4]
 * "Block Diffusion"): encoder pass over d_block_ids (int32[canvas]) at the
 * committed length, then length += canvas. DG_ERR_CAPACITY if it does not fit. */
int dg_commit_block(dg_ctx* ctx, const int32_t* d_block_ids, void* stream);

/* One layer on a caller-provided fp32 residual d_x [rows x d_model] (in/out),
 * rows <= max(canvas, prefill_rows), attending to cache [0, length) plus the rows (causal or
 * not); the rows' K/V are written at [length, length + rows); length is not
 * changed. */
int dg_forward_layer(dg_ctx* ctx, int32_t layer, float* d_x, int32_t rows, int32_t causal,
                     void* stream);

/* Native denoising loop of one canvas ([P4] "Reverse diffusion process" and
 * "Two-Fold Adaptive Stopping"): dg_init_canvas, then for step = 0 ..
 * max_steps-1: dg_denoise_step (self-conditioned on the previous step),
 * dg_sample_canvas, and a 16-byte copy of the stop state into a pinned host
 * slot of the context; the block is the final step's argmax, copied to
 * d_block_out (int32[canvas]); with commit != 0 it is then committed.
 * d_logits: [canvas x vocab] caller scratch. *steps_out (host) receives the
 * number of steps run. The calling thread waits for a step's copy only when
 * that step could have stopped: the stable count is 0 on step 0 and grows by
 * at most one a step, so under the two-fold rule a step whose count cannot
 * have reached stable_needed cannot stop, and the next step is queued behind
 * it without waiting (with DG_SCHED_STOP_EITHER every step is waited for). No
 * step after the stopping one is launched. */
int dg_generate_block(dg_ctx* ctx, const dg_sched* sched, int32_t block, void* d_logits,
                      int32_t* d_block_out, int32_t commit, int32_t* steps_out, void* stream);

/* Device addresses of context buffers, for inspection by tests and tools. */
enum {
  DG_BUF_X = 0,             /* float [canvas x d_model] residual stream */
  DG_BUF_H = 1,             /* dtype [canvas x d_model] RMSNorm of the residual
                               stream (after a layer: of the layer's output) */
  DG_BUF_ROUTER_LOGITS = 2, /* float [canvas x n_experts] (last layer run) */
  DG_BUF_SEL = 3,           /* int32 [canvas x top_k] selected experts */
  DG_BUF_GATE = 4,          /* float [canvas x top_k] gates */
  DG_BUF_SC = 5,            /* float [canvas x d_model] self-conditioning vector */
  DG_BUF_CANVAS = 6,        /* int32 [canvas] loop canvas */
  DG_BUF_PRED = 7,          /* int32 [canvas] loop argmax */
  DG_BUF_STOP = 8,          /* dg_stop_state of the loop */
  DG_BUF_ENTROPY = 9,       /* float [canvas] */
  DG_BUF_ROW_STATS = 10,    /* float [canvas x 2] */
  DG_BUF_ACCEPT = 11,       /* uint8 [canvas] */
  DG_BUF_Q = 12,            /* dtype [canvas x n_q_heads*head_dim] queries (last layer run) */
  DG_BUF_ATTN = 13,         /* dtype [canvas x n_q_heads*head_dim] attention output */
  DG_BUF_SHARED_ACT = 14,   /* dtype [canvas x d_shared] shared-expert hidden activation */
  DG_BUF_SLOT_OUT = 15,     /* float [canvas*top_k x d_model] gated routed-expert outputs, expert-major slots */
  DG_BUF_SLOT_OF = 16,      /* int32 [canvas x top_k] slot of each (row, choice) */
  DG_BUF_SEL_LAYERS = 17,   /* int32 [n_layers][R][top_k], R = max(canvas, prefill_rows): the experts every
                               layer chose for the rows of the last pass (a denoising step, or the last
                               chunk of a prefill / commit, whose last layer computes only K and V) */
  DG_BUF_OFFSETS = 18       /* int32 [2 n_experts + 1] (last layer run): the experts' first slots and the
                               slot count, then the experts by decreasing token count (lower index
                               first on ties), the order the routed-expert launches take them in */
};
int dg_ctx_buffer(const dg_ctx* ctx, int32_t which, void** d_ptr, size_t* bytes);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
