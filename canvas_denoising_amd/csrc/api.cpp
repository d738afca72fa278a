// C ABI of libdg: argument validation and dispatch to the HIP launchers.
// Every check runs before anything is enqueued, so a rejected call has no
// side effect.
#include <math.h>

#include <string>

#include "dg_common.h"

namespace dg {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int hip_check(hipError_t e, const char* what) {
  return fail(DG_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// launchers (sampler.hip, synth.hip)
size_t sample_workspace_bytes(int64_t rows, int64_t vocab);
int launch_init_canvas(uint64_t seed, int block, int n, int vocab, int32_t* canvas, dg_stop_state* stop,
                       hipStream_t stream);
int launch_sample(const void* logits, int dtype, int rows, int vocab, float temp, const dg_sched& sc, int step,
                  int block, int32_t* canvas, int32_t* pred, uint8_t* accept, float* entropy, float* row_stats,
                  dg_stop_state* stop, void* ws, hipStream_t stream);
int launch_synth_normal(uint64_t seed, uint64_t tid, int64_t n, float sigma, int dtype, void* out, hipStream_t s);
int launch_synth_ids(uint64_t seed, uint64_t tid, int64_t n, int vocab, int32_t* out, hipStream_t s);
int launch_synth_logits(uint64_t seed, int step, int rows, int vocab, float sigma, float peak, void* out,
                        hipStream_t s);
int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks, hipStream_t s);
size_t static_scratch_bytes();
int static_scratch(void** out);

float temperature(const dg_sched& s, int step) {
  const double t0 = s.t_start, t1 = s.t_end;
  if (s.max_steps <= 1) return static_cast<float>(t0);
  return static_cast<float>(t0 + (t1 - t0) * (static_cast<double>(step) / (s.max_steps - 1)));
}

int check_sched(const dg_sched* s, int step) {
  if (s == nullptr) return fail(DG_ERR_INVALID, "sched is NULL");
  if (s->max_steps < 1) return fail(DG_ERR_INVALID, "max_steps must be >= 1");
  if (!(s->t_start > 0.f) || !(s->t_end > 0.f) || !isfinite(s->t_start) || !isfinite(s->t_end))
    return fail(DG_ERR_INVALID, "temperatures must be finite and > 0");
  if (!isfinite(s->entropy_bound) || !isfinite(s->stop_mean_entropy))
    return fail(DG_ERR_INVALID, "entropy thresholds must be finite");
  if (s->stable_needed < 0) return fail(DG_ERR_INVALID, "stable_needed must be >= 0");
  if ((s->mode & ~(DG_SCHED_STOP_EITHER | DG_SCHED_ACCEPT_GROUP | DG_SCHED_SAMPLE)) != 0)
    return fail(DG_ERR_INVALID, "unknown sched mode flag");
  if (step < 0 || step >= s->max_steps) return fail(DG_ERR_INVALID, "step outside [0, max_steps)");
  return DG_OK;
}

int check_sample_args(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab, const dg_sched* sched,
                             int32_t step, int32_t block, const int32_t* d_canvas, const int32_t* d_pred,
                             const dg_stop_state* d_stop) {
  if (int rc = check_sched(sched, step)) return rc;
  if (dtype != DG_BF16 && dtype != DG_F32) return fail(DG_ERR_INVALID, "dtype must be DG_BF16 or DG_F32");
  if (rows < 1 || rows > 65535) return fail(DG_ERR_SHAPE, "rows must be in [1, 65535]");
  if (vocab < 1) return fail(DG_ERR_SHAPE, "vocab must be >= 1");
  if (block < 0) return fail(DG_ERR_INVALID, "block must be >= 0");
  if (!d_logits || !d_canvas || !d_pred || !d_stop)
    return fail(DG_ERR_INVALID, "d_logits, d_canvas, d_pred and d_stop are required");
  if (reinterpret_cast<uintptr_t>(d_logits) % 16 != 0) return fail(DG_ERR_INVALID, "d_logits must be 16-byte aligned");
  return DG_OK;
}

}  // namespace dg

using namespace dg;

extern "C" {

const char* dg_last_error(void) { return g_last_error.c_str(); }

const char* dg_version(void) { return "libdg 0.1 (gfx950)"; }

float dg_temperature(const dg_sched* sched, int32_t step) {
  if (sched == nullptr) return NAN;
  return temperature(*sched, step);
}

size_t dg_sample_workspace_size(int32_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  return sample_workspace_bytes(rows, vocab);
}

int dg_init_canvas(const dg_sched* sched, int32_t block, int32_t canvas, int32_t vocab, int32_t* d_canvas,
                   dg_stop_state* d_stop, void* stream) {
  if (int rc = check_sched(sched, 0)) return rc;
  if (block < 0) return fail(DG_ERR_INVALID, "block must be >= 0");
  if (canvas < 1 || canvas > 65536) return fail(DG_ERR_SHAPE, "canvas must be in [1, 65536]");
  if (vocab < 1) return fail(DG_ERR_SHAPE, "vocab must be >= 1");
  if (d_canvas == nullptr) return fail(DG_ERR_INVALID, "d_canvas is NULL");
  return launch_init_canvas(sched->seed, block, canvas, vocab, d_canvas, d_stop, as_stream(stream));
}

int dg_sample_canvas(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab, const dg_sched* sched,
                     int32_t step, int32_t block, int32_t* d_canvas, int32_t* d_pred, uint8_t* d_accept,
                     float* d_entropy, float* d_row_stats, dg_stop_state* d_stop, void* d_workspace,
                     size_t ws_bytes, void* stream) {
  if (int rc = check_sample_args(d_logits, dtype, rows, vocab, sched, step, block, d_canvas, d_pred, d_stop))
    return rc;
  if (!d_workspace) return fail(DG_ERR_INVALID, "d_workspace is required");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256 != 0)
    return fail(DG_ERR_INVALID, "d_workspace must be 256-byte aligned");
  if (ws_bytes < sample_workspace_bytes(rows, vocab)) return fail(DG_ERR_CAPACITY, "sampler workspace too small");
  const float T = temperature(*sched, step);
  return launch_sample(d_logits, dtype, rows, vocab, T, *sched, step, block, d_canvas, d_pred, d_accept, d_entropy,
                       d_row_stats, d_stop, d_workspace, as_stream(stream));
}

int dg_sample_canvas_static(const void* d_logits, int32_t dtype, int32_t rows, int32_t vocab, const dg_sched* sched,
                            int32_t step, int32_t block, int32_t* d_canvas, int32_t* d_pred, uint8_t* d_accept,
                            float* d_entropy, float* d_row_stats, dg_stop_state* d_stop, void* stream) {
  if (int rc = check_sample_args(d_logits, dtype, rows, vocab, sched, step, block, d_canvas, d_pred, d_stop))
    return rc;
  if (sample_workspace_bytes(rows, vocab) > static_scratch_bytes())
    return fail(DG_ERR_CAPACITY, "rows x vocab need more than the 1 MiB static sampler scratch (use dg_sample_canvas)");
  void* ws = nullptr;
  if (int rc = static_scratch(&ws)) return rc;
  const float T = temperature(*sched, step);
  return launch_sample(d_logits, dtype, rows, vocab, T, *sched, step, block, d_canvas, d_pred, d_accept, d_entropy,
                       d_row_stats, d_stop, ws, as_stream(stream));
}

int dg_synth_normal(uint64_t seed, uint64_t tid, int64_t n, float sigma, int32_t dtype, void* d_out, void* stream) {
  if (n < 0) return fail(DG_ERR_SHAPE, "n must be >= 0");
  if (dtype != DG_BF16 && dtype != DG_F32) return fail(DG_ERR_INVALID, "bad dtype");
  if (n > 0 && d_out == nullptr) return fail(DG_ERR_INVALID, "d_out is NULL");
  if (!isfinite(sigma) || sigma < 0.f) return fail(DG_ERR_INVALID, "sigma must be finite and >= 0");
  return launch_synth_normal(seed, tid, n, sigma, dtype, d_out, as_stream(stream));
}

int dg_synth_uniform_ids(uint64_t seed, uint64_t tid, int64_t n, int32_t vocab, int32_t* d_out, void* stream) {
  if (n < 0 || vocab < 1) return fail(DG_ERR_SHAPE, "n must be >= 0 and vocab >= 1");
  if (n > 0 && d_out == nullptr) return fail(DG_ERR_INVALID, "d_out is NULL");
  return launch_synth_ids(seed, tid, n, vocab, d_out, as_stream(stream));
}

int dg_stream_read(const void* d_src, int64_t bytes, uint32_t* d_sink, int32_t blocks, void* stream) {
  if (!d_src || !d_sink) return fail(DG_ERR_INVALID, "d_src and d_sink are required");
  if (bytes < 16 || bytes % 16 != 0) return fail(DG_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(d_src) % 16 != 0) return fail(DG_ERR_INVALID, "d_src must be 16-byte aligned");
  if (blocks < 1 || blocks > (1 << 20)) return fail(DG_ERR_INVALID, "blocks must be in [1, 2^20]");
  return launch_stream_read(d_src, bytes, d_sink, blocks, as_stream(stream));
}

int dg_synth_planted_logits(uint64_t seed, int32_t step, int32_t rows, int32_t vocab, float sigma, float peak,
                            void* d_out, void* stream) {
  if (rows < 0 || vocab < 1 || step < 0) return fail(DG_ERR_SHAPE, "rows >= 0, vocab >= 1, step >= 0 required");
  if (rows > 0 && d_out == nullptr) return fail(DG_ERR_INVALID, "d_out is NULL");
  if (!isfinite(sigma) || !isfinite(peak)) return fail(DG_ERR_INVALID, "sigma and peak must be finite");
  return launch_synth_logits(seed, step, rows, vocab, sigma, peak, d_out, as_stream(stream));
}

}  // extern "C"
