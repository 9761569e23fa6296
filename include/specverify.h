/*
 * libspecverify -- the verify-and-speculate step of speculative decoding and
 * of speculative speculative decoding (SSD), for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  No C++ or framework types cross it: plain pointers, sizes and the
 * small structs below.  Unless stated otherwise every array pointer is a
 * DEVICE pointer owned by the caller; the library allocates no memory of its
 * own (sv_verify_noalloc aside, whose workspace is a static device array),
 * launches only on the stream it is given (a hipStream_t passed as
 * void*, NULL = the default stream) and returns before the work completes:
 * results are valid once the caller has synchronised that stream.  Its
 * process-wide state is a per-device cache of launch sizing (CU count and
 * kernel occupancy, queried once per device and never changed afterwards)
 * and, for sv_verify_noalloc only, that array and its address on each
 * device; calls from several host threads are safe (sv_verify_noalloc's
 * calls on one device share its array: see there).
 *
 * What is computed (sources are cited by page title and section):
 *
 *  - A small drafter proposes k tokens; the target scores all of them in one
 *    forward pass, keeps the correct prefix and regenerates from the first
 *    divergence ("How It Works", speculative-sampling project page,
 *    sourcepulse.org project 1842340; "What changes in SSD", hysenlabs.com
 *    editorial on SSD).  The rule is speculative sampling in its textbook
 *    form (the same page names the Google and DeepMind variants under
 *    "Highlighted Details"): accept drafted token d at position j iff
 *    u < min(1, p_j(d) / q_j(d)); at the first rejection n emit a token drawn
 *    by inverse CDF from the normalised residual max(0, p_n - q_n); if all k
 *    are accepted emit a bonus token drawn from p_k.  The result is exact:
 *    the emitted tokens follow the target distribution ("What changes in
 *    SSD").
 *  - p and q are the softmax of the logits at the sequence's temperature;
 *    at temperature 0 the step is greedy (argmax, lowest id on ties), the
 *    sampler's greedy/stochastic switch in the tanishqkumar/ssd repository
 *    summary (thehardwarestore.ai, highlighted sampler file).
 *  - SSD's forked recovery tokens: per position, the top-f draft tokens with
 *    the drafted token masked out, so the drafter can pre-speculate every
 *    likely verification outcome (same summary, highlighted async-SD
 *    utilities file; f alternatives in the SSD README's benchmark commands,
 *    m.111cn.net translation, section 基准测试).
 *
 * Shapes and layout.  B sequences (B <= 8192 and B * (k + 1) <= 32768 per
 * call), k drafted positions (1 <= k <= 63),
 * positions j = 0..k where j = k is the bonus position, vocabulary
 * 2 <= V <= 1048576 shared by target and drafter (speculative-sampling page, "Quick Start &
 * Requirements": both models must share one vocabulary).  Logits are
 * [B][k+1][V] with V contiguous, addressed with element strides; every row
 * start must be 16-byte aligned (so strides must be multiples of 4 fp32 /
 * 8 bf16 elements).  Uniforms are caller-supplied in [0, 1): the library
 * holds no random-number state.
 *
 * Numerics.  Elementwise exponentials in fp32, per-row sums accumulated in
 * fp32 within a lane and in fp64 across lanes and chunks, acceptance ratios
 * and CDF prefixes in fp64.  Reductions have a fixed order: results are
 * bitwise deterministic from run to run.
 *
 * Errors.  Host-detectable problems (null required pointers, sizes out of
 * range, misaligned rows, unknown dtype, short workspace) return a status and
 * launch nothing.  Problems visible only in device data make the affected
 * sequence an error: a temperature that is NaN, negative or infinite, a
 * drafted id outside [0, V), or a logits row that is read and whose maximum
 * is not finite (+inf, or every entry -inf).  Such a sequence gets -1 in its
 * integer outputs and NaN in its float outputs; nothing is read out of
 * bounds.  NaN logits are outside the contract (results unspecified, still
 * in bounds).
 *
 * Workspace.  Every compute call takes a device workspace of at least
 * sv_workspace_size() bytes.  It must be zero-filled once, before its first
 * use (sv_workspace_init, or any zero fill).  Its arrival counters sit in a
 * control header at its start, at offsets that depend on no size, and every
 * call that runs to completion returns them to zero, so one workspace then
 * serves any sequence of calls of any entry point and any sizes.  Calls
 * that share a workspace must not overlap in time (use one workspace per
 * stream).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1, /* null required pointer, size out of range, bad enum */
  SV_ERR_MISALIGNED = 2,  /* a logits or output row does not start 16-byte aligned */
  SV_ERR_WORKSPACE = 3,   /* workspace null or smaller than sv_workspace_size() */
  SV_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* One batch of verify inputs.  target/draft: [B][k+1][V] logits of dtype
 * `dtype` at the given element strides (row k of the draft is read only for
 * forks; a draft of [B][k][V] may be passed with forks off).
 * draft_tokens: [B][k] int32, contiguous.  temperature: [B] fp32; 0 =
 * greedy. */
typedef struct sv_batch {
  int32_t B, k, V;
  int32_t dtype; /* sv_dtype, same for target and draft */
  const void* target;
  int64_t t_seq_stride, t_row_stride;
  const void* draft;
  int64_t d_seq_stride, d_row_stride;
  const int32_t* draft_tokens;
  const float* temperature;
} sv_batch;

/* Forked recovery outputs: tokens [B][k+1][f] int32 (required), probs
 * [B][k+1][f] fp32 (nullable), 1 <= f <= min(16, V-1).  Probabilities are
 * the softmax at the sequence temperature of the draft logits with the
 * drafted token masked out (nothing masked at j = k); (1, 0, ...) at
 * temperature 0.
 * hits [B] int32 (nullable; sv_verify only, ignored by sv_forked_topf):
 * the speculation-cache lookup of each sequence's outcome, as computed by
 * sv_cache_hit from this call's forks, accept_len and out_token. */
typedef struct sv_forks {
  int32_t f;
  int32_t* tokens;
  float* probs;
  int32_t* hits;
} sv_forks;

/* Optional per-call extras.  ev_stats_begin / ev_stats_end: hipEvent_t
 * handles (as void*) recorded on the call's stream immediately before and
 * after the streaming statistics kernel, for timing it on its own; NULL =
 * not recorded. */
typedef struct sv_opts {
  void* ev_stats_begin;
  void* ev_stats_end;
} sv_opts;

/* Bytes of workspace any entry point needs for these sizes (an upper bound
 * over dtypes).  For sv_softmax_temp pass B = rows, k = 0, f = 0.
 * Returns 0 for sizes out of range. */
size_t sv_workspace_size(int32_t B, int32_t k, int32_t V, int32_t f);

/* Zero-fills `bytes` bytes of a workspace on `stream` with a fill kernel
 * (no memset node, so it can be captured in a graph).  Needed once per
 * workspace, before its first use. */
sv_status sv_workspace_init(void* ws, size_t bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sv_status_string(int32_t status);

/* Library version string (static storage). */
const char* sv_version(void);

/* Temperature softmax of `rows` logits rows, the p and q of the
 * speculative-sampling rule at the sequence's temperature (the sampler's
 * temperature, tanishqkumar/ssd repository summary, highlighted sampler
 * file; the rule itself: "How It Works", speculative-sampling project
 * page):
 * probs[r][t] = softmax(logits[r] / tau)[t] with tau = temperature[r /
 * rows_per_temp]; one-hot at the first maximum when tau = 0.  logits: rows
 * of V elements at row_stride elements; probs: fp32 rows at out_row_stride
 * elements (16-byte aligned rows).  A row whose maximum is not finite, or
 * whose temperature is invalid, comes back as NaN.  Reads the logits twice
 * (statistics, then normalise-and-write). */
sv_status sv_softmax_temp(const void* logits, int32_t dtype, int64_t rows,
                          int32_t V, int64_t row_stride,
                          const float* temperature, int64_t rows_per_temp,
                          float* probs, int64_t out_row_stride, void* ws,
                          size_t ws_bytes, void* stream);

/* The verify step ("How It Works", speculative-sampling project page; the
 * target checks all drafted tokens in one pass and keeps the accepted
 * prefix, "What changes in SSD", hysenlabs.com editorial): acceptance tests
 * u < min(1, p/q), first rejection, and the recovery or bonus draw, with the
 * forked recovery tokens (async-SD utilities file, tanishqkumar/ssd
 * repository summary) fused into the same pass over the draft logits when
 * `forks` is non-NULL.
 *   u_accept [B][k]    uniform of the acceptance test at each position
 *   u_recover [B][k+1] uniform of the draw at the outcome position n
 *   accept_len [B]     out: n = number of accepted drafted tokens, in [0, k]
 *   out_token [B]      out: the recovery token (n < k) or bonus token (n = k)
 *   p_draft, q_draft [B][k] out (nullable): p_j(d_j), q_j(d_j) (one-hot
 *                      indicators at temperature 0).  Passing q_draft makes
 *                      the draft rows be read also at temperature 0.
 * Launches: a streaming statistics kernel (one resident round of waves,
 * each over an equal slab range of one row, writing per-range partials),
 * then a decision kernel that merges the partials per row, decides each
 * sequence, ranks the forks, re-reads only row n of the temperature > 0
 * sequences for the draw and, with forks->hits, writes the lookup of
 * sv_cache_hit once the token and the forks are in (no third launch). */
sv_status sv_verify(const sv_batch* in, const float* u_accept,
                    const float* u_recover, int32_t* accept_len,
                    int32_t* out_token, float* p_draft, float* q_draft,
                    const sv_forks* forks, void* ws, size_t ws_bytes,
                    void* stream);

/* sv_verify with extras (see sv_opts); opts may be NULL. */
sv_status sv_verify_ex(const sv_batch* in, const float* u_accept,
                       const float* u_recover, int32_t* accept_len,
                       int32_t* out_token, float* p_draft, float* q_draft,
                       const sv_forks* forks, void* ws, size_t ws_bytes,
                       void* stream, const sv_opts* opts);

/* Bytes of the static scratch array of sv_verify_noalloc, on each device it
 * runs on (enough for B = 64, k = 7, V = 151936, f <= 16). */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* sv_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  Same
 * arguments, outputs, launches and results as sv_verify, bitwise, without
 * the workspace arguments: the workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES, one per device, held from the first call on a
 * device until the process ends.  The call allocates and frees nothing.
 *   Returns SV_ERR_WORKSPACE, launching nothing, when the shape needs more
 *   than that (sv_workspace_size(B, k, V, f) > SV_NOALLOC_SCRATCH_BYTES).
 *   The first call on a device looks up the array's address with that
 *   device current and zero-fills the array on `stream` (one extra launch);
 *   make that first call outside a graph capture.  Every call on a device
 *   uses the same array and leaves its contents behind: calls on one device
 *   that may overlap in time (several streams, several threads) race and
 *   must be serialised by the caller, for example by issuing them all on
 *   one stream. */
sv_status sv_verify_noalloc(const sv_batch* in, const float* u_accept,
                            const float* u_recover, int32_t* accept_len,
                            int32_t* out_token, float* p_draft, float* q_draft,
                            const sv_forks* forks, void* stream);

/* The draw at a given position of each sequence, and optionally the full
 * residual distributions: the regeneration from the first divergence of
 * "How It Works" (speculative-sampling project page), from the normalised
 * residual max(0, p_n - q_n) whose use keeps the output law the target's
 * ("What changes in SSD", hysenlabs.com editorial).
 *   position [B]   n in [0, k]: n < k draws from max(0, p_n - q_n)
 *                  normalised (p_n if that is zero everywhere), n = k draws
 *                  the bonus token from p_k; greedy at temperature 0
 *   u_recover [B][k+1]; token_out [B] out
 *   residual [B][k+1][V] fp32 out (nullable): for every position j < k the
 *                  normalised residual, p_k at j = k, one-hot at the target
 *                  argmax at temperature 0; rows at res_seq_stride /
 *                  res_row_stride elements, 16-byte aligned.
 * A position outside [0, k] makes that sequence an error. */
sv_status sv_residual_sample(const sv_batch* in, const int32_t* position,
                             const float* u_recover, int32_t* token_out,
                             float* residual, int64_t res_seq_stride,
                             int64_t res_row_stride, void* ws,
                             size_t ws_bytes, void* stream);

/* Forked recovery tokens alone, from the draft logits only: the top-f
 * tokens per position with the drafted token masked (async-SD utilities
 * file, tanishqkumar/ssd repository summary; f alternatives per position,
 * SSD README translation, m.111cn.net, section 基准测试), for drafter-side
 * use in SSD, where the drafter runs on its own device without the target's
 * logits ("What changes in SSD", hysenlabs.com editorial).  in->target may
 * be NULL. */
sv_status sv_forked_topf(const sv_batch* in, const sv_forks* forks, void* ws,
                         size_t ws_bytes, void* stream);

/* Speculation-cache lookup of verification outcomes.  In SSD the drafter
 * speculates ahead of time for the likely outcomes of verification and a
 * correct guess is returned at once ("What changes in SSD", hysenlabs.com
 * editorial); the forked recovery tokens are the guesses, and they decide
 * cache hits and misses (tanishqkumar/ssd repository summary, async-SD
 * utilities file).  The outcome of sequence b is (n, t) = (accept_len[b],
 * out_token[b]); the drafter speculated, at position n, for the f tokens
 * fork_tokens[b][n][0..f-1].
 *   fork_tokens [B][k+1][f] int32, accept_len [B], out_token [B] (device,
 *                 caller-owned; e.g. the outputs of sv_verify, or forks
 *                 from an earlier sv_forked_topf on the drafter's side)
 *   hits [B] int32 out: the index r with fork_tokens[b][n][r] == t (the
 *                 first, if tokens repeat), else -1; -1 also when n is
 *                 outside [0, k] or t < 0 (an error outcome).
 * 1 <= k <= 63, 1 <= f <= 16, B >= 0.  One small kernel; no workspace. */
sv_status sv_cache_hit(int32_t B, int32_t k, int32_t f,
                       const int32_t* fork_tokens, const int32_t* accept_len,
                       const int32_t* out_token, int32_t* hits, void* stream);

/* The drafter's own draw from its logits rows: greedy or stochastic by
 * temperature (tanishqkumar/ssd repository summary, highlighted sampler
 * file).  tokens[r] = the lowest id holding the maximum of row r when its
 * temperature is 0; otherwise the inverse-CDF draw from softmax(row / tau)
 * with the uniform uniforms[r]: the first token, in id order, whose running
 * sum of probabilities exceeds the uniform (the last token of positive
 * probability if rounding leaves none).
 *   logits       rows of V elements (dtype) at row_stride elements; rows
 *                16-byte aligned; V <= 1048576 (fp32) / 2097152 (bf16)
 *   temperature  [ceil(rows / rows_per_temp)] fp32: row r uses
 *                temperature[r / rows_per_temp]
 *   uniforms     [rows] fp32 in [0, 1)
 *   tokens       [rows] int32 out; -1 for a row whose maximum is not finite
 *                or whose temperature is NaN, negative or infinite.
 * One block per row reads the row once (plus one 1-2 KiB slab of it for
 * the draw); no workspace. */
sv_status sv_sample_temp(const void* logits, int32_t dtype, int64_t rows,
                         int32_t V, int64_t row_stride,
                         const float* temperature, int64_t rows_per_temp,
                         const float* uniforms, int32_t* tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
