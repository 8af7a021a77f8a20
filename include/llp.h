/*
 * llp.h -- C ABI of the fused linear log-prob operator for AMD Instinct MI355X (gfx950).
 *
 * The operator turns a language model's final hidden states and its (vocabulary-partitioned)
 * output projection into per-token log-probabilities of given target ids, optional entropy,
 * their gradients, the rank-ordered merge of per-shard partials, and compact top-p replay
 * scores. Sources (three pull-request pages; cited by title and section):
 *   [CUDA provider] "feat(rl-kernel): add CUDA linear logp provider integration"
 *   [ROCm provider] "feat(rl-kernel): add ROCm linear logp provider integration"
 *   [top-p replay]  "Perf/cuda compact top p replay"
 *
 * The request structs mirror the provider contract of [CUDA provider, "Changes" /
 * "Linear-logp provider contract"]: a request (LinearLogpRequest) carrying a projection
 * (LinearProjection: output-layer hidden states, local projection weight and bias), a
 * vocabulary partition (VocabPartition: tensor-parallel vocabulary range, real and padded
 * vocabulary sizes) and a token layout (TokenLayout: packing and loss masks), plus target
 * ids and the temperature.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; the caller owns all memory
 *     and keeps it valid until the work enqueued on `stream` completes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Execution calls (forward, merge, backward, top_p_replay) never allocate, never
 *     synchronize and never read device memory on the host, so they can be captured into a
 *     HIP graph. Every row's result is a function of that row's inputs and the fixed kernel
 *     configuration only: results are bitwise reproducible run to run and do not depend on
 *     how rows are batched or ordered (dweight/dbias: reproducible for a fixed batch).
 *   - Errors are returned as llp_status; no exception crosses the ABI and the library never
 *     aborts. llp_last_error() describes the last non-OK status of the calling thread.
 *   - Host-detectable problems (shapes, strides, alignment, partition, temperature, limits)
 *     return LLP_ERR_INVALID_ARGUMENT before anything is enqueued. Data-dependent problems
 *     found on the device (a bad target or replay id, a malformed cu_seqlens) are OR-ed into
 *     the optional device `status_word` (LLP_STATUS_* bits) and the affected rows get -inf
 *     log-probabilities; nothing becomes NaN.
 */
#ifndef LLP_H
#define LLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLP_API __attribute__((visibility("default")))

#define LLP_VERSION "0.1.0"
/* Most replay candidate ids per row ([top-p replay, "Changes" table]: up to 64 ids). */
#define LLP_MAX_REPLAY_IDS 64
/* Most vocabulary shards llp_merge combines in one call. */
#define LLP_MAX_WORLD 64

/* Return codes. Only llp_open returns LLP_ERR_UNAVAILABLE: that is the one status a caller
 * may treat as "provider unavailable, use another path" ([CUDA provider, "Motivation"]:
 * auto mode falls back only on an explicit unavailable report; strict mode fails closed).
 * Loading (llp_open) is kept apart from execution so that an execution failure is never
 * mistaken for unavailability ([CUDA provider], review discussion). */
typedef enum {
  LLP_OK = 0,
  LLP_ERR_UNAVAILABLE = 1,      /* no gfx950 device / kernels cannot be loaded (llp_open) */
  LLP_ERR_INVALID_ARGUMENT = 2, /* malformed request; nothing was enqueued */
  LLP_ERR_UNSUPPORTED = 3,      /* well formed but outside the compiled envelope */
  LLP_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  LLP_ERR_INTERNAL = 5
} llp_status;

/* Device status-word bits (OR-ed with integer atomics). */
enum {
  LLP_STATUS_TARGET_OUT_OF_RANGE = 1, /* a scored row's target is outside [0, real_vocab) */
  LLP_STATUS_TARGET_NOT_FOUND = 2,    /* no shard (or no replay candidate) holds the target */
  LLP_STATUS_REPLAY_ID_INVALID = 4,   /* a replay id outside [-1, real_vocab) (slot ignored) */
  LLP_STATUS_LAYOUT_INVALID = 8       /* cu_seqlens not 0 = c0 <= c1 <= ... <= cS = T */
};

enum { LLP_DTYPE_BF16 = 1, LLP_DTYPE_F32 = 2 };
enum { LLP_OP_FORWARD = 1, LLP_OP_BACKWARD = 2 };
/* Request flags.
 *   LLP_FLAG_WANT_ENTROPY     the forward also computes the entropy.
 *   LLP_FLAG_OVERWRITE_GRADS  llp_backward writes dweight and dbias (= this call's gradient,
 *                             padding rows 0) instead of adding to them: the first chunk of a
 *                             step needs no zeroed buffer and no read of one. Ignored by
 *                             llp_forward.
 *   LLP_FLAG_G_SLABS          llp_backward never holds the whole G: it computes G, its
 *                             dhidden and dweight products one vocabulary slab of
 *                             LLP_G_SLAB_COLUMNS local columns at a time, in slab order, and
 *                             adds each slab's dhidden into fp32 partials in the workspace.
 *                             The workspace holds one slab of G instead of all of it
 *                             (llp_workspace_bytes sizes it from this flag). dweight and dbias
 *                             are bitwise those of the default mode; dhidden agrees to rounding
 *                             (its vocabulary sum runs slab by slab) and is still bitwise
 *                             reproducible and independent of the batch. Ignored by
 *                             llp_forward. */
enum { LLP_FLAG_WANT_ENTROPY = 1, LLP_FLAG_OVERWRITE_GRADS = 2, LLP_FLAG_G_SLABS = 4 };
#define LLP_G_SLAB_COLUMNS 32768

/* Library identity and route evidence ([CUDA provider, "Changes"]: validation of identity;
 * native/provider route evidence). */
typedef struct {
  char name[32];       /* "lm_head_linear_logp_amd" */
  char version[16];    /* LLP_VERSION */
  char arch[32];       /* device architecture the kernels run on, e.g. "gfx950" */
  char route[128];     /* kernel variant and tile configuration */
  int32_t max_replay_ids;
  int32_t num_cus;
  int32_t device;
  int32_t reserved;
} llp_info;

/* LinearProjection ([CUDA provider, "Megatron integration"]: output-layer hidden states, local
 * projection weight and bias).
 *   hidden  [T, H] bf16, row stride hidden_stride (elements, >= H, multiple of 8), 16-byte
 *           aligned base.
 *   weight  [local_size, H] bf16 -- this shard's rows of the LM-head weight, row stride
 *           weight_stride (elements, >= H, multiple of 8), 16-byte aligned base. Rows past the
 *           shard's real columns (padding) are never read into a result.
 *   bias    [local_size] of bias_dtype (LLP_DTYPE_BF16 or LLP_DTYPE_F32), or NULL; 16-byte
 *           aligned base for F32, 8-byte for BF16.
 *   H must be a positive multiple of 64, at most 2^20 (else LLP_ERR_UNSUPPORTED). Operand
 *   rows are addressed with 32-bit byte offsets, which bounds the envelope (else
 *   LLP_ERR_UNSUPPORTED): hidden_stride and weight_stride < 2^23, T * hidden_stride * 2 < 2^31
 *   (the bytes the T hidden rows span), T <= 2^23 - 256 and local_size <= 2^23 - 256. */
typedef struct {
  const void* hidden;
  int64_t hidden_stride;
  const void* weight;
  int64_t weight_stride;
  const void* bias;
  int32_t bias_dtype;
  int32_t reserved;
  int64_t hidden_size; /* H */
} llp_projection;

/* VocabPartition ([CUDA provider, "Megatron integration"]: tensor-parallel vocabulary range
 * and real/padded vocabulary sizes; [CUDA provider, "CUDA compatibility and launch support"]:
 * tensor parallelism is the vocabulary reduction group). The shard owns global ids
 * [offset, offset + local_size); its real columns are the first
 * clamp(real_vocab - offset, 0, local_size). Requires 0 <= offset, offset + local_size <=
 * padded_vocab, 0 < real_vocab <= padded_vocab, 0 <= rank < world <= LLP_MAX_WORLD, and for
 * world == 1: offset == 0 and local_size == padded_vocab. local_size == 0 is an empty shard. */
typedef struct {
  int64_t offset;
  int64_t local_size;
  int64_t real_vocab;
  int64_t padded_vocab;
  int32_t rank;
  int32_t world;
} llp_vocab_partition;

/* TokenLayout ([CUDA provider, "Summary"]: the framework keeps token layout and masking;
 * [CUDA provider, "CUDA compatibility and launch support"]: context parallelism is row
 * ownership). Rows are independent: num_seqs/cu_seqlens describe packing and are validated
 * on the device (LLP_STATUS_LAYOUT_INVALID) but do not change any row's arithmetic.
 *   num_tokens  T >= 0 rows (llp_forward / llp_backward: at most 2^23 - 256, else
 *               LLP_ERR_UNSUPPORTED; llp_forward_logits: below 2^31, else INVALID_ARGUMENT).
 *   cu_seqlens  int32 [num_seqs + 1] device array or NULL (num_seqs ignored when NULL).
 *   loss_mask   uint8 [T] device array (non-zero = scored) or NULL (every row scored).
 * Unscored rows are not computed; all their outputs are written as 0 and they get no
 * gradient. Targets are row-aligned: the operator never shifts them. */
typedef struct {
  int64_t num_tokens;
  int32_t num_seqs;
  int32_t reserved;
  const int32_t* cu_seqlens;
  const uint8_t* loss_mask;
} llp_token_layout;

/* LinearLogpRequest ([CUDA provider, "Motivation"]: logits or projection, target ids,
 * tensor-parallel group, token layout and masks).
 *   target_ids   int64 [T] device array (global vocabulary ids).
 *   temperature  finite, > 0. Logits are z = (hidden . weight^T + bias) * fl32(1/temperature):
 *                temperature is applied exactly once ([ROCm provider, "Megatron
 *                integration"]; [top-p replay, "Summary"]).
 *   flags        LLP_FLAG_WANT_ENTROPY, LLP_FLAG_OVERWRITE_GRADS, LLP_FLAG_G_SLABS.
 *   status_word  int32 device word OR-ed with LLP_STATUS_* bits, or NULL. */
typedef struct {
  llp_projection proj;
  llp_vocab_partition vocab;
  llp_token_layout layout;
  const int64_t* target_ids;
  float temperature;
  uint32_t flags;
  int32_t* status_word;
} llp_request;

/* Per-shard partials, one value per row, all device arrays of length T.
 * Written by llp_forward and llp_top_p_replay, read by llp_merge.
 *   target_logit  z[target] if the target lies in this shard's real columns, else 0
 *   in_range      1 if it does, else 0
 *   lse           log-sum-exp of z over the shard's real columns (-inf for no columns)
 *   entropy       entropy of the shard-local softmax (0 for no columns); NULL = not wanted
 *   logp          target_logit - lse if in_range, else -inf; NULL = not wanted.
 *                 For an unsharded call (world == 1) this is the final log-probability.
 * Unscored rows: every field 0. */
typedef struct {
  float* target_logit;
  uint8_t* in_range;
  float* lse;
  float* entropy;
  float* logp;
} llp_partials;

/* Merged per-row results of llp_merge (device arrays of length T; entropy may be NULL). */
typedef struct {
  float* logp;
  float* lse;
  float* entropy;
} llp_final_out;

/* Inputs of llp_backward (device arrays of length T).
 *   lse       the merged (global) log-sum-exp of every row (llp_merge / llp_forward at world 1)
 *   dlogp     upstream gradient of each row's logp
 *   dentropy  upstream gradient of each row's entropy, or NULL
 *   entropy   the merged entropy (required when dentropy is given) */
typedef struct {
  const float* lse;
  const float* dlogp;
  const float* dentropy;
  const float* entropy;
} llp_bwd_in;

/* Outputs of llp_backward.
 *   dhidden  bf16 [T, H], row stride dhidden_stride (>= H, multiple of 8): OVERWRITTEN with
 *            this shard's contribution G . weight (unscored rows 0). With world > 1 the caller
 *            sums the shards' dhidden.
 *   dweight  fp32 [local_size, H], row stride dweight_stride (>= H, multiple of 4, < 2^21,
 *            else INVALID_ARGUMENT / UNSUPPORTED), 16-byte aligned base: ACCUMULATED (+=) with
 *            G^T . hidden over this call's rows; padding rows untouched. With
 *            LLP_FLAG_OVERWRITE_GRADS: OVERWRITTEN with G^T . hidden, padding rows (and every
 *            row of a call with no rows) written as 0; bitwise the accumulate form applied
 *            to a zeroed buffer.
 *   dbias    fp32 [local_size] ACCUMULATED (OVERWRITTEN with LLP_FLAG_OVERWRITE_GRADS), or
 *            NULL.
 * G[t, v] = (dlogp_t (1[v = target_t] - p_tv) - dentropy_t p_tv (z_tv - E_p z_t)) / temperature
 * with p = exp(z - lse), is rounded to bf16 once and feeds all three products. */
typedef struct {
  void* dhidden;
  int64_t dhidden_stride;
  float* dweight;
  int64_t dweight_stride;
  float* dbias;
} llp_bwd_out;

/* Compact top-p replay request ([top-p replay, "Summary"]: replay the native finite nucleus,
 * scoring the compact replay ids directly instead of a full-vocabulary keep mask;
 * [top-p replay, "Changes" table]: validate replay inputs, sort and deduplicate up to 64 ids,
 * apply temperature, return local reductions).
 *   logits        [T, local_size] this shard's local logits (logits_dtype: LLP_DTYPE_F32 or
 *                 LLP_DTYPE_BF16), row stride logits_stride elements.
 *   num_tokens    T rows, 0 <= T < 2^31 (else LLP_ERR_INVALID_ARGUMENT).
 *   replay_ids    int64 [T, num_replay] global ids, row stride replay_stride; -1 = empty slot;
 *                 num_replay in [1, LLP_MAX_REPLAY_IDS]. Duplicates count once.
 *   processed_logprobs must be 1: replay scores processed (temperature/top-p) log-probs
 *                 only; raw mode is rejected ([top-p replay], review: replay only for
 *                 processed logprobs).
 * Writes target_logit, in_range, lse and logp of `out` (entropy must be NULL). */
typedef struct {
  const void* logits;
  int32_t logits_dtype;
  int32_t num_replay;
  int64_t logits_stride;
  int64_t num_tokens;
  llp_vocab_partition vocab;
  const int64_t* replay_ids;
  int64_t replay_stride;
  const int64_t* target_ids;
  const uint8_t* loss_mask;
  float temperature;
  int32_t processed_logprobs;
  int32_t* status_word;
} llp_topp_request;

/* Logits-input forward request ([CUDA provider, "Megatron integration"]: strict LM-head local
 * logits are reused when available, avoiding a second projection; [top-p replay, "Summary"]:
 * temperature is applied exactly once).
 *   logits        [T, local_size] of logits_dtype (LLP_DTYPE_F32 or LLP_DTYPE_BF16), the
 *                 shard's unscaled local logits h . W^T + b; row stride logits_stride
 *                 (elements, >= local_size; the rows must be 16-byte aligned: base aligned and
 *                 stride * element size a multiple of 16). Padded columns are never read.
 *   vocab, layout, target_ids, temperature, flags, status_word: as in llp_request (z = x *
 *                 fl32(1/temperature); flags: LLP_FLAG_WANT_ENTROPY). */
typedef struct {
  const void* logits;
  int32_t logits_dtype;
  int32_t reserved;
  int64_t logits_stride;
  llp_vocab_partition vocab;
  llp_token_layout layout;
  const int64_t* target_ids;
  float temperature;
  uint32_t flags;
  int32_t* status_word;
} llp_logits_request;

/* Dense keep-mask replay request ([top-p replay, "Changes" table]: the local logits are
 * reused with a keep mask and excluded entries are -inf; [top-p replay, "Validation"]: the
 * dense-mask and compact forms agree bitwise across shard offsets and empty shards).
 *   logits        as in llp_topp_request, with 16-byte aligned rows (see llp_logits_request).
 *   keep_mask     uint8 [num_tokens, local_size], row stride keep_stride (bytes, >= local_size,
 *                 multiple of 16), 16-byte aligned base; nonzero = the column is in the row's
 *                 nucleus. Columns past the shard's real ones are ignored.
 *   num_tokens, vocab, target_ids, loss_mask, temperature, processed_logprobs, status_word:
 *                 as in llp_topp_request. */
typedef struct {
  const void* logits;
  int32_t logits_dtype;
  int32_t processed_logprobs;
  int64_t logits_stride;
  const uint8_t* keep_mask;
  int64_t keep_stride;
  int64_t num_tokens;
  llp_vocab_partition vocab;
  const int64_t* target_ids;
  const uint8_t* loss_mask;
  float temperature;
  int32_t reserved;
  int32_t* status_word;
} llp_keep_mask_request;

/* Loading phase: checks that `device` is a gfx950 GPU and loads the kernels on it; fills
 * `info` (may be NULL). Returns LLP_ERR_UNAVAILABLE when there is no such device. Must
 * succeed on the current device before any execution call. Idempotent. */
LLP_API llp_status llp_open(int32_t device, llp_info* info);

/* Workspace bytes an execution call needs for `req` and `op` (LLP_OP_FORWARD or
 * LLP_OP_BACKWARD): a pure function of the shapes (and, for the backward, of
 * LLP_FLAG_G_SLABS). The caller allocates it (device memory, 256-byte aligned) and passes it
 * to that call. */
LLP_API llp_status llp_workspace_bytes(const llp_request* req, int32_t op, size_t* bytes);

/* Fused forward for one shard: per row, z over the shard's real columns, lse, the target
 * logit, optional entropy and the local logp, without materializing [T, V] logits
 * ([top-p replay, "Changes" table]: fused linear-logp kernel; [CUDA provider, "Motivation"]).
 * Writes every non-NULL field of `out` (target_logit, in_range and lse are required; entropy
 * only with LLP_FLAG_WANT_ENTROPY). */
LLP_API llp_status llp_forward(const llp_request* req, const llp_partials* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* llp_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * workspace is a static device array of the library, 32 MiB on every device the library is
 * opened on, held until the process ends; the call allocates nothing. Results are bitwise
 * those of llp_forward (the same kernels).
 *   Limit: llp_workspace_bytes(req, LLP_OP_FORWARD) must be at most 32 MiB, else
 *   LLP_ERR_UNSUPPORTED before anything is enqueued: e.g. up to 4608 rows over a 151669-column
 *   shard, or 18432 over a 37984-column one.
 *   Every call on one device shares that device's array. Calls that overlap on a device (on
 *   different streams, or from several threads without ordering) race and give wrong results:
 *   serialize them. No part of the array needs to start at zero (a call writes every value it
 *   reads before reading it), so nothing is cleared between calls. */
LLP_API llp_status llp_forward_noalloc(const llp_request* req, const llp_partials* out,
                                       void* stream);

/* Rank-ordered merge of `world` shards' partials ([top-p replay, "Summary"]: rank-ordered
 * reductions, shards with no candidates handled). `parts` is a HOST array of `world` structs
 * in rank order whose fields are device arrays of length num_tokens (entropy NULL in every
 * part = no merged entropy). Per row: lse = M + log sum_r exp(lse_r - M) over non-empty
 * shards; logp = target_logit of the first shard holding the target minus lse, or -inf
 * (LLP_STATUS_TARGET_NOT_FOUND); entropy = sum_r exp(lse_r - lse)(entropy_r + lse - lse_r).
 * loss_mask (device, may be NULL) zeroes unscored rows. out->entropy may be NULL.
 * 0 <= num_tokens < 2^31 (else LLP_ERR_INVALID_ARGUMENT). */
LLP_API llp_status llp_merge(int32_t world, const llp_partials* parts, int64_t num_tokens,
                             const uint8_t* loss_mask, const llp_final_out* out,
                             int32_t* status_word, void* stream);

/* Backward for one shard: dhidden = G . weight (overwrite), dweight += G^T . hidden,
 * dbias += sum_t G (= instead of += with LLP_FLAG_OVERWRITE_GRADS) (gradients must flow: [CUDA provider, "Motivation"], strict mode rejects
 * detached gradients). Needs the merged lse of every scored row. */
LLP_API llp_status llp_backward(const llp_request* req, const llp_bwd_in* in,
                                const llp_bwd_out* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Compact top-p replay scoring for one shard (see llp_topp_request). Follow with llp_merge
 * over the shards for the final log-probability. */
LLP_API llp_status llp_top_p_replay(const llp_topp_request* req, const llp_partials* out,
                                    void* stream);

/* Logits-input forward for one shard: the partials of llp_forward (target_logit, in_range,
 * lse required; entropy with LLP_FLAG_WANT_ENTROPY; logp optional) from the shard's local
 * logits instead of hidden states and weight. Needs no workspace. */
LLP_API llp_status llp_forward_logits(const llp_logits_request* req, const llp_partials* out,
                                      void* stream);

/* Dense keep-mask replay scoring for one shard: the partials of llp_top_p_replay (entropy must
 * be NULL) for the nucleus given as a keep mask. For a nucleus of at most LLP_MAX_REPLAY_IDS
 * ids the results are bitwise those of llp_top_p_replay given the same ids. */
LLP_API llp_status llp_keep_mask_replay(const llp_keep_mask_request* req,
                                        const llp_partials* out, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
LLP_API const char* llp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LLP_H */
