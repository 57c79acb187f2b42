/* spec_verify.h -- C ABI of the MI355X (gfx950) verify-and-resample library
 * for speculative sampling.
 *
 * What one call computes (for each of B sequences, independently):
 *   - the target model's K_b+1 logit rows and the draft model's K_b logit
 *     rows are turned into "adjusted distributions" q_t (target) and p_t
 *     (draft): temperature, then one filter (plain, top-k, nucleus or
 *     greedy), applied before the rejection step and to both models
 *     (paperlayer.ai summary of arXiv 2302.01318, section "Modified
 *     Rejection Sampling"; FDE Interviews breakdown, section 01);
 *   - draft token d_t is kept with probability min(1, q_t(d_t)/p_t(d_t)),
 *     left to right; q is the target and p the draft (FDE Interviews
 *     breakdown, section 01 and its figure "The idea, visually");
 *   - at the first rejection n a replacement is drawn from the normalised
 *     positive part of q_n - p_n and the rest of the draft is discarded;
 *     if all K_b drafts survive, one more token is drawn from the target's
 *     last logit row (same sources; roadtointelligence.com "Speculative
 *     Decoding", section "Draft, then verify", with its letters swapped);
 *   - each sequence therefore emits between 1 and K_b+1 tokens.
 *
 * Random numbers come from Philox4x32-10 (Salmon et al., SC'11) keyed by
 * `seed`, with counter (g lo, t, purpose, g hi), g = row_offset + b, and
 * purposes ACCEPT = 0, RESAMPLE = 1, BONUS = 2.  The uniform is
 * (word0 >> 8) * 2^-24.  Results are a pure function of the inputs, the seed
 * and g, so a batch may be split across calls or devices with row_offset.
 *
 * Threading and streams: a handle serves one stream at a time; use one
 * handle per concurrently used stream.  spec_verify_run is asynchronous on
 * the given stream, allocates nothing and never synchronises.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sv_handle_s* sv_handle_t;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Filter applied to both models' rows (after temperature, before the
 * rejection step).
 *   SV_PLAIN : softmax(x / tau) over every token whose logit is not -inf.
 *   SV_TOPK  : keep every token whose raw logit is >= the k-th largest raw
 *              logit of the row (ties at the boundary are all kept), then
 *              softmax(x / tau) over the kept set.
 *   SV_TOPP  : nucleus.  Tokens are grouped by equal logit and visited in
 *              descending order of probability under softmax(x / tau); a
 *              group is kept iff the mass of the groups before it is
 *              < top_p (the first group is always kept; top_p = 1 keeps
 *              every token of non-zero probability); renormalised.
 *   SV_GREEDY: one-hot at the lowest index among the maximal raw logits;
 *              the temperature is ignored. */
typedef enum { SV_PLAIN = 0, SV_TOPK = 1, SV_TOPP = 2, SV_GREEDY = 3 } sv_mode;

/* Return codes (synchronous argument errors launch nothing). */
enum {
  SV_OK = 0,
  SV_EINVAL = -1,    /* bad pointer, size or default parameter            */
  SV_ECAPACITY = -2, /* B > max_batch or K_max > max_k                    */
  SV_EDTYPE = -3,    /* unknown dtype                                      */
  SV_EHIP = -4,      /* a HIP runtime call failed; see last_error          */
  SV_ENOMEM = -5     /* workspace allocation failed at create              */
};

/* row_status bits, written per sequence by the device.  Bits 0, 1, 2 and 6
 * are errors: the sequence then has accepted = -1 and every out_token -1.
 * The others are informational. */
enum {
  SV_ST_TOKEN = 1u << 0,         /* a draft token d_t (t < K_b) is outside [0, V)   */
  SV_ST_NONFINITE = 1u << 1,     /* a used logit is NaN or +inf                    */
  SV_ST_EMPTY = 1u << 2,         /* every logit of a used row is -inf               */
  SV_ST_ZERO_RESIDUAL = 1u << 3, /* (q-p)+ had no mass (rounding): drew from q_n    */
  SV_ST_PZERO = 1u << 4,         /* a tested draft token had p_t(d_t) = 0           */
  SV_ST_MARGIN = 1u << 5,        /* a device-side decision was within 1e-6 of its
                                    boundary (an accept ratio, a CDF boundary or a
                                    nucleus cumulative mass)                        */
  SV_ST_PARAM = 1u << 6,         /* invalid per-row parameter (K_b, mode, tau, k,
                                    top_p)                                          */
  SV_ST_FULLSELECT = 1u << 7,    /* a top-k/top-p threshold needed the full-row
                                    selection (slow path)                           */
  SV_ST_REREAD = 1u << 8,        /* the final draw re-read full logit rows           */
  SV_ST_LOCATED = 1u << 9        /* that draw read only the span or chunk located by
                                    sums made before it (the span sums of a spread
                                    residual draw, or the chunk sums of a plain
                                    target row for its bonus draw)                  */
};

/* Create-time capacity.  vocab is fixed for the handle; 1 <= vocab <= 2^22,
 * max_batch >= 1, 0 <= max_k <= 64.  device is the HIP device ordinal. */
typedef struct {
  int32_t max_batch;
  int32_t max_k;
  int32_t vocab;
  int32_t dtype; /* sv_dtype */
  int32_t device;
} sv_config;

/* Per-call arguments.  Every pointer is a device pointer on the handle's
 * device; the caller owns all of them and keeps them alive until the work
 * on the stream has finished.  All arrays are dense and row-major.
 *
 *   target_logits [B][K_max+1][V]  dtype of the handle.  Target position t
 *                                  scores draft slot t; position K_b is the
 *                                  bonus position.  Rows t > K_b are never
 *                                  read (padding may hold anything).
 *   draft_logits  [B][K_max][V]    rows t >= K_b are never read.  May be NULL
 *                                  when K_max = 0, or when every sequence is
 *                                  greedy (mode NULL, default_mode
 *                                  SV_GREEDY): greedy verification needs only
 *                                  the target's argmax, so then only the
 *                                  K_b + 1 target rows are read; diag's p
 *                                  column is NaN and SV_ST_ZERO_RESIDUAL /
 *                                  SV_ST_PZERO, which need the draft's
 *                                  argmax, are never set.
 *   draft_tokens  [B][K_max] int32 may be NULL when K_max = 0.
 *   k_per_row     [B] int32 in [0, K_max], or NULL (every row uses K_max).
 *   mode          [B] uint8 sv_mode, or NULL (default_mode).
 *   temperature   [B] float > 0, or NULL (default_temperature).
 *   top_k         [B] int32 in [1, V], or NULL (default_top_k).
 *   top_p         [B] float in (0, 1], or NULL (default_top_p).
 *   seed, row_offset: see the RNG note above.
 * Outputs:
 *   accepted      [B] int32: n in [0, K_b], or -1 for an error row.
 *   out_tokens    [B][K_max+1] int32: d_0..d_{n-1}, then the resampled or
 *                                  bonus token, then -1.
 *   row_status    [B] uint32 SV_ST_* bits, or NULL.
 *   diag          [B][K_max][2] float: (q_t(d_t), p_t(d_t)) for t < K_b,
 *                                  NaN elsewhere and on error rows; or NULL.
 * B = 0 is a no-op.
 * The library trusts the caller's buffers: target_logits must hold
 * B * (K_max + 1) * vocab elements and draft_logits B * K_max * vocab
 * elements of the handle's dtype (vocab is the row stride), and the index
 * arrays the sizes above.  A shorter buffer is read out of bounds; nothing
 * on the device can detect it.
 * Rows longer than 4096 bf16 / 2048 fp32 logits must be whole 16-byte
 * vectors: vocab * element size a multiple of 16 and both logit buffers
 * 16-byte aligned; otherwise validation returns SV_EINVAL (shorter rows
 * may be unaligned). */
typedef struct {
  int32_t B;
  int32_t K_max;
  const void* target_logits;
  const void* draft_logits;
  const int32_t* draft_tokens;
  const int32_t* k_per_row;
  const uint8_t* mode;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t default_mode;
  float default_temperature;
  int32_t default_top_k;
  float default_top_p;
  uint64_t seed;
  uint64_t row_offset;
  int32_t* accepted;
  int32_t* out_tokens;
  uint32_t* row_status;
  float* diag;
} sv_args;

/* Creates a handle for cfg->device and allocates its device workspace
 * (hipMalloc).  On success *out receives the handle and SV_OK is returned;
 * on failure *out is NULL and a negative code is returned. */
int spec_verify_create(sv_handle_t* out, const sv_config* cfg);

/* Enqueues the whole step on `stream` (a hipStream_t; NULL is the null
 * stream).  Validates the arguments on the host first (see
 * spec_verify_validate) and returns a negative code without launching
 * anything if they are invalid.  Data errors found on the device are
 * reported per sequence through row_status.  No allocation, no host
 * synchronisation.  The call may be captured into a HIP graph (stream
 * capture): its kernels become graph nodes that read the argument pointers
 * given at capture, so each replay uses the data then in those buffers, and
 * replays must not overlap other runs of the same handle.  Stage profiling
 * is skipped under capture. */
int spec_verify_run(sv_handle_t h, const sv_args* args, void* stream);

/* If any run was enqueued or captured through h, waits for the device to
 * finish all queued work (which includes every such run and any launch of a
 * graph holding one), then frees the workspace and the handle.  The wait is
 * device-wide by design: a run records no event and allocates nothing, so
 * the handle does not know which streams its runs used, and a device
 * synchronisation is the one wait that covers them all; it also waits for
 * work of other handles and other libraries on the device.  A graph
 * holding a captured run must not be launched after its handle is
 * destroyed.  NULL is accepted. */
int spec_verify_destroy(sv_handle_t h);

/* Host-only check of a (config, args) pair: pointer presence, sizes
 * against the capacity, default parameters that some row may use.  Makes no
 * HIP call and dereferences no device pointer. */
int spec_verify_validate(const sv_config* cfg, const sv_args* args);

/* Bytes of device workspace spec_verify_create allocates for cfg, or 0 if
 * cfg is invalid.  Host-only. */
uint64_t spec_verify_workspace_bytes(const sv_config* cfg);

/* Stage timing, for measurement.  After spec_verify_profile_begin(h, n),
 * the next n calls of spec_verify_run on h record HIP events on their own
 * stream for the two stages of the first launch batch (a call is one batch
 * unless it exceeds 2^23 logit rows or 2^22 sequences): stage 0 is the
 * streaming pass over the logit rows with each row's finish (statistics,
 * threshold, kept list), stage 1 the per-sequence accept walk and draw.  Each stage is timed from the start to the end of its
 * kernels' own dispatches (events attached to the dispatch, so the launch
 * gap before a kernel is not counted).  The events are created here, so run
 * still allocates nothing; runs under stream capture record none.  spec_verify_profile_end waits for the
 * last recorded event, writes the summed milliseconds of stage i to ms[i]
 * for i < min(n_stages, 2), releases the events and returns the number of
 * calls recorded (negative code on error).  Calling begin again discards an
 * unfinished profile. */
int spec_verify_profile_begin(sv_handle_t h, int max_calls);
int spec_verify_profile_end(sv_handle_t h, double* ms, int n_stages);

/* Streaming ceiling, for measurement: reads the first floor(bytes / 8192)
 * whole 8 KB blocks at data (a 16-byte aligned device pointer) once, with
 * the streaming pass's chunk (one 8 KB block per wave, 16-byte vectors,
 * constant offsets, non-temporal loads) and no arithmetic beyond an xor
 * fold, on the given stream (NULL = the default stream), asynchronously.
 * One wave per block: the grid is as large as the data.  out is a device
 * pointer to at least 4 bytes; it is written only when the fold hits a
 * fixed value.  Allocates nothing.  Returns SV_OK, or SV_EINVAL / SV_EHIP
 * with spec_verify_last_error set.  It computes nothing of the method: it
 * gives the read rate the streaming pass is measured against. */
int spec_verify_stream_probe(const void* data, size_t bytes, void* out, void* stream);

/* One point of a read-rate sweep, for measurement: reads the first
 * floor(bytes / (loads_per_lane * 1024)) whole blocks at data (16-byte
 * aligned) once, a block being 64 lanes x loads_per_lane 16-byte vectors,
 * with a persistent grid of waves_per_cu * 256 waves in work-groups of 4.
 * Work-group g takes the g-th of equal contiguous ranges of blocks, its
 * waves take the range's blocks in turn, and each wave keeps its next
 * block's loads in flight while it folds the current one (non-temporal
 * loads, an xor fold).  loads_per_lane is 4, 8 or 16; waves_per_cu is 1 to
 * 32.  data, out and stream as for spec_verify_stream_probe; asynchronous,
 * allocates nothing.  Returns SV_OK, or SV_EINVAL (a NULL or unaligned
 * pointer, a parameter out of range: nothing is launched) / SV_EHIP, with
 * spec_verify_last_error set.  Sweeping both parameters gives the read rate
 * of the memory system apart from any one access pattern. */
int spec_verify_stream_probe_sweep(const void* data, size_t bytes, int loads_per_lane, int waves_per_cu, void* out,
                                   void* stream);

/* The step's random numbers, for verification: writes to out[i] (device
 * memory, n words) word 0 of Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * SC'11) at key `seed` and counter (g[i] low 32 bits, t[i], purpose[i],
 * g[i] high 32 bits) -- the word from which run takes each uniform as
 * (word >> 8) / 2^24, with g the sequence's global index (row_offset + b),
 * t its position and purpose 0 (accept test), 1 (resample) or 2 (bonus).
 * g, t and purpose are device arrays of n entries; n >= 0.  Asynchronous on
 * `stream`, allocates nothing.  Returns SV_OK, or SV_EINVAL (a NULL array
 * with n > 0, n negative: nothing is launched) / SV_EHIP, with
 * spec_verify_last_error set.  It lets a test compare the device generator
 * with an independent one word for word. */
int spec_verify_philox_words(uint64_t seed, const uint64_t* g, const uint32_t* t, const uint32_t* purpose,
                             int64_t n, uint32_t* out, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Runs the
 * same step as spec_verify_run with the same kernels and results, on
 * cfg->device and `stream`, with no handle: the workspace is a static
 * device buffer of SV_STATIC_SCRATCH_BYTES that the library holds on each
 * device it runs on until the process ends.  cfg gives V, the dtype and the
 * device; max_batch and max_k only bound B and K_max as in
 * spec_verify_validate.  A call whose workspace (which grows with B,
 * K_max and V) exceeds the buffer returns SV_ECAPACITY, launches nothing
 * and says how many bytes it needed in spec_verify_last_error.  No
 * allocation, no synchronisation, no events.  Every call on one device
 * shares that device's buffer: calls that overlap on a device (other
 * streams, other threads, graph replays) race and give wrong results;
 * order them on one stream.  The buffer needs no clearing between calls:
 * each call writes every workspace entry it reads, except the arrival
 * counters of rows streamed in parts and of fused sequence steps, which
 * are zero when the library's code loads and which every call that
 * completes leaves at zero. */
#define SV_STATIC_SCRATCH_BYTES ((uint64_t)64 << 20)
int spec_verify_run_static(const sv_config* cfg, const sv_args* args, void* stream);

/* Text of the last error reported on the calling thread ("" if none). */
const char* spec_verify_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
