/*
 * specverify.h -- C ABI of the batched speculative-sampling verify step
 * (hand-written HIP kernels for gfx950 / MI355X).
 *
 * Pages cited (all about speculative decoding):
 *   [WR] wrblog.cn, "推测解码：草稿模型、接受率、正确性与加速边界"
 *   [RL] rainlin-net.pages.dev, "投机解码" (notes)
 *   [BS] baisen.site, "投机采样 / 投机解码（Speculative Decoding）"
 *   [MN] magicnetworld.com, "投机解码到底能加速多少：把接受率、草稿成本与墙钟收益算清楚"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees or retains caller memory and keeps no
 *   state between calls, apart from the optional profiling hook
 *   (spec_set_stage_timer), the allocation-free call's per-GPU scratch, and
 *   a side stream with two events per (device, caller stream), made on the
 *   first call that uses one (the statistics with a dense q and Z', and the
 *   draft-logits calls under top-k or top-p) and kept until the process
 *   ends (at most 64 such pairs; past that, and where one cannot be made,
 *   the work stays on the caller's stream).  All
 *   scratch lives in the caller's `workspace`
 *   (device memory of at least the reported workspace size, 16-byte
 *   aligned, contents need not be initialised).
 * - Layout is contiguous row-major.  `target_logits` is [B, gamma+1, V]
 *   (float32 or bfloat16, see sv_dtype); `draft_probs` (q) is [B, gamma, V]
 *   float32; `draft_ids` is [B, gamma] int32 (the ragged calls take packed
 *   tensors instead, described with them).  The logits and q base pointers
 *   must be 16-byte aligned.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  The returned status reports only synchronous host-side
 *   validation and launch errors; outputs are valid once the stream reaches
 *   the end of the call.  Calls that share a workspace must not overlap.
 * - Argument errors return a status and launch nothing.  Data faults never
 *   abort: they raise per-request bits in `out_row_flags` (SV_ROW_*).
 * - Inputs are read-only.  Every output element is written on every call.
 * - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations have int as their underlying type in C++ too, so every
 * int a caller passes for one is a value of that type; the library checks
 * the value and returns SV_ERR_INVALID_ARG for one it does not know. */
#ifdef __cplusplus
#define SV_ENUM_INT : int
#else
#define SV_ENUM_INT
#endif

typedef enum SV_ENUM_INT {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size or parameter */
  SV_ERR_UNSUPPORTED = 2, /* a size the kernels do not handle (e.g. V >= 2^31) */
  SV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  SV_ERR_HIP = 4          /* a kernel launch failed                           */
} sv_status;

typedef enum SV_ENUM_INT { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Decoding rules that turn target logits into the processed distribution p
 * ([WR] §2.3: p is the distribution after the production decoding rules;
 * [WR] §7.2 temperature, §7.3 top-k / top-p).  Order: temperature, top-k on
 * the logits (every token tied with the k-th largest logit is kept), top-p on
 * the renormalised top-k distribution (the smallest most-probable prefix whose
 * mass reaches top_p, plus tokens tied with its last one), renormalise.
 *   temperature : finite, > 0
 *   top_k       : 0 or >= V disables; otherwise 1 <= top_k < V
 *   top_p       : in (0, 1]; 1 disables                                     */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
} sv_sampling_params;

/* Per-request status bits in out_row_flags. */
#define SV_ROW_BAD_ID 1u       /* a draft id outside [0, V) was rejected        */
#define SV_ROW_Q_ZERO 2u       /* q(d)=0 at an evaluated position: accepted iff p(d)>0 */
#define SV_ROW_Z_DEGENERATE 4u /* rejected with an empty residual; token drawn from p */
#define SV_ROW_NONFINITE 8u    /* NaN/+Inf logits (or an all -Inf row), or q(d) NaN,
                                  negative or +Inf: no token emitted              */
#define SV_ROW_EOS 16u         /* ragged calls: an end-of-sequence token was emitted */
#define SV_ROW_BAD_SPAN 32u    /* ragged calls: the request's draft span is out of order,
                                  out of range or longer than gamma_max: no token
                                  emitted                                          */

/* Bytes of workspace that spec_verify_sample, spec_verify_greedy,
 * spec_accept_stats, spec_verify_sample_stats, spec_verify_sample_lenient
 * and (with gamma = gamma_max) the ragged calls need for these sizes (the
 * maximum over them).  Returns 0 when the sizes are invalid. */
size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int32_t V, sv_dtype dt,
                                  sv_sampling_params prm);

/* Sampling verify ([WR] §6 multi-token verification; [RL] §1 steps 3-4;
 * [BS] §四 rules (1)-(2)).
 * For each request b, position j = 0..gamma-1 in order:
 *   accept d_j iff u_accept[b,j] < p_j(d_j) / q_j(d_j)   ([WR] §4.1)
 *   (q_j(d_j) = 0: accept iff p_j(d_j) > 0, SV_ROW_Q_ZERO);
 * stop at the first rejection j*: emit d_0..d_{j*-1}, then a token drawn from
 * the residual (p_{j*} - q_{j*})_+ ([WR] §5; [RL] §2); if every draft passes,
 * emit all gamma drafts and a bonus token drawn from p_gamma ([WR] §6).
 * A draw takes the first token id (ascending) whose running sum of weights
 * exceeds u_resample[b, n_accepted] * (sum of weights).
 *   target_logits  [B, gamma+1, V]  dt
 *   draft_probs    [B, gamma, V]    float32, the draft's processed q (not
 *                                   renormalised by the library)
 *   draft_ids      [B, gamma]       int32
 *   u_accept       [B, gamma]       float32 in [0, 1)
 *   u_resample     [B, gamma+1]     float32 in [0, 1); only index n_accepted is used
 *   out_tokens       [B, gamma+1]   int32: emitted tokens, -1 padded
 *   out_num_accepted [B]            int32 in [0, gamma]; emitted = n + 1 ([WR] §10)
 *   out_row_flags    [B]            uint32 SV_ROW_* bits, or NULL
 * gamma = 0 is plain sampling from p_0.  B = 0 is a no-op. */
sv_status spec_verify_sample(const void* target_logits, sv_dtype dt, const float* draft_probs,
                             const int32_t* draft_ids, const float* u_accept,
                             const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                             sv_sampling_params prm, int32_t* out_tokens,
                             int32_t* out_num_accepted, uint32_t* out_row_flags,
                             void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify_sample without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing.  Its
 * scratch is a static device array of SV_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its address
 * is looked up on the first call on each device).  Sizes whose workspace
 * (spec_verify_workspace_size) exceeds it return SV_ERR_UNSUPPORTED and
 * launch nothing; SV_ERR_HIP when the array's address cannot be obtained.
 * Every call on one GPU shares that array, so calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Arguments, outputs and results are those of spec_verify_sample. */
#define SV_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
sv_status spec_verify_sample_noalloc(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                     const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                     int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm,
                                     int32_t* out_tokens, int32_t* out_num_accepted, uint32_t* out_row_flags,
                                     void* stream);

/* Greedy verify ([WR] §7.1; [RL] §2 last paragraph; [BS] §二 example):
 * g_j = argmax of row j (lowest id on ties), j = 0..gamma;
 * n = first j < gamma with d_j != g_j (else gamma); emit d_0..d_{n-1}, g_n.
 * A request whose logits hold NaN emits nothing (SV_ROW_NONFINITE). */
sv_status spec_verify_greedy(const void* target_logits, sv_dtype dt, const int32_t* draft_ids,
                             int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                             int32_t* out_num_accepted, uint32_t* out_row_flags,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Acceptance statistics of positions j = 0..gamma-1 (rows j of the same
 * [B, gamma+1, V] logits; the bonus row is not read):
 *   out_alpha       = sum_x min(p_j, q_j)          ([WR] §4.2; [MN] §三)
 *   out_z_pq        = sum_x (p_j - q_j)_+  (residual mass Z)     ([RL] §2)
 *   out_z_qp        = sum_x (q_j - p_j)_+                        ([BS] §五)
 *   out_accept_prob = min(1, p_j(d_j) / q_j(d_j))  ([WR] §6)
 * each [B, gamma] float32, or NULL (not computed).  q is used as given.
 * q_j(d_j) = 0 gives accept_prob 1 if p_j(d_j) > 0 else 0; an id outside
 * [0, V) gives NaN; a non-finite logits row gives NaN in all four outputs of
 * that position.  Cost: out_z_qp needs sum_x q_j(x) over the whole row, a
 * pass over q; without it, a position whose p_j is truncated to a kept set
 * reads q only at that set's ids (p_j is 0 elsewhere, so alpha and z_pq are
 * sums over the set). */
sv_status spec_accept_stats(const void* target_logits, sv_dtype dt, const float* draft_probs,
                            const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V,
                            sv_sampling_params prm, float* out_alpha, float* out_z_pq,
                            float* out_z_qp, float* out_accept_prob, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Sampling verify and acceptance statistics together: the outputs of
 * spec_verify_sample and of spec_accept_stats for the same inputs, from one
 * pass over the target logits (the statistics reuse the sampling call's row
 * results for rows 0..gamma-1 instead of recomputing them).  Arguments are
 * those of the two calls; each statistics output may be NULL, as in
 * spec_accept_stats.  Workspace: spec_verify_workspace_size (which covers this
 * call).  [WR] §4.2 and §6; [RL] §2; [MN] §三 (acceptance rate, monitored per
 * round to adapt gamma: [MN] §九, point 3). */
sv_status spec_verify_sample_stats(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                   const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                   int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, int32_t* out_tokens,
                                   int32_t* out_num_accepted, uint32_t* out_row_flags, float* out_alpha,
                                   float* out_z_pq, float* out_z_qp, float* out_accept_prob, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---- q formed in the library from the draft's logits -----------------------
 * [WR] §2.3 and [MN] §二 (notation): q, like p, is the distribution after the
 * decoding rules.  These calls take the draft model's logits instead of q and
 * form q_j with the same rules and the same parameters as p_j (temperature,
 * top-k on the logits, top-p on the renormalised top-k distribution,
 * renormalise), then verify or measure exactly as the calls above do with
 * that q.
 *   draft_logits [B, gamma, V]  draft_dt (float32 or bfloat16), contiguous,
 *                               16-byte aligned base; read-only.
 * A draft row holding NaN or +Inf (or all -Inf) has no q: it reads as a NaN
 * q row, so a valid draft id at that position makes the request
 * SV_ROW_NONFINITE (as a NaN q(d) does above), and the statistics of that
 * position are NaN.  A draft id outside the draft's own kept set has
 * q(d) = 0 (SV_ROW_Q_ZERO rules).
 * The workspace holds both the target's and the draft rows' intermediate
 * results; size it with spec_verify_draft_logits_workspace_size (0 for
 * invalid sizes).  Everything else (outputs, errors, streams, determinism)
 * is as for spec_verify_sample / spec_accept_stats. */
size_t spec_verify_draft_logits_workspace_size(int32_t B, int32_t gamma, int32_t V, sv_dtype dt,
                                               sv_dtype draft_dt, sv_sampling_params prm);

sv_status spec_verify_sample_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                          sv_dtype draft_dt, const int32_t* draft_ids, const float* u_accept,
                                          const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                                          sv_sampling_params prm, int32_t* out_tokens, int32_t* out_num_accepted,
                                          uint32_t* out_row_flags, void* workspace, size_t workspace_bytes,
                                          void* stream);

sv_status spec_accept_stats_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                         sv_dtype draft_dt, const int32_t* draft_ids, int32_t B, int32_t gamma,
                                         int32_t V, sv_sampling_params prm, float* out_alpha, float* out_z_pq,
                                         float* out_z_qp, float* out_accept_prob, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* ---- lenient acceptance -------------------------------------------------------
 * [MN] §八 (lenience): the draft distribution is scaled to beta * q before it
 * is compared with the target, so d_j is accepted iff
 *   u_accept[b,j] < p_j(d_j) / (lenience * q_j(d_j)),
 * a looser test that is no longer lossless: a token is emitted with at most
 * 1/lenience times its target probability.  The pages give no replacement
 * rule for this variant; the one taken here keeps the step with beta * q in
 * place of q, so a rejection draws from (p_j - lenience * q_j)_+ (which keeps
 * that bound).  lenience must be in (0, 1]; 1 gives exactly spec_verify_sample.
 * Everything else (layout, outputs, flags, workspace) is as for
 * spec_verify_sample. */
sv_status spec_verify_sample_lenient(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                     const int32_t* draft_ids, const float* u_accept, const float* u_resample,
                                     int32_t B, int32_t gamma, int32_t V, sv_sampling_params prm, float lenience,
                                     int32_t* out_tokens, int32_t* out_num_accepted, uint32_t* out_row_flags,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---- ragged batches: a draft length per request ----------------------------
 * [WR] §11.2 and [MN] §九 (point 3): no single draft length suits every
 * request, so gamma is chosen per request and one verify batch holds
 * requests with different gamma_b (0 <= gamma_b <= gamma_max).  The inputs
 * are packed, with no padding rows:
 *   cu_draft     [B + 1]              int32 DEVICE array, cu_draft[0] = 0,
 *                                     non-decreasing, cu_draft[B] = n_draft;
 *                                     gamma_b = cu_draft[b+1] - cu_draft[b]
 *   draft_ids    [n_draft]            int32, request b's at cu_draft[b] ..
 *   draft_probs  [n_draft, V]         float32 q rows, same positions
 *   u_accept     [n_draft]            float32, same positions
 *   target_logits [n_draft + B, V]    request b's gamma_b + 1 rows start at
 *                                     row cu_draft[b] + b
 *   u_resample   [n_draft + B]        float32, same rows as the logits
 * n_draft (a host value) must equal cu_draft[B] and be <= B * gamma_max.
 * Outputs are padded: out_tokens [B, gamma_max + 1] (-1 after the emitted
 * tokens), out_num_accepted [B], out_row_flags [B].  A request whose span is
 * out of order, out of range or longer than gamma_max is not read: it emits
 * nothing and is flagged SV_ROW_BAD_SPAN.  gamma_b = 0 is plain sampling.
 *
 * End of sequence ([WR] §14.3: no token is committed after an EOS).  With
 * eos_id >= 0, verification also stops at an accepted draft equal to
 * eos_id: that draft is the last emitted token (at slot n_accepted, so
 * n_accepted counts the drafts before it) and no token is drawn.  Any
 * emitted EOS (an accepted draft, a replacement or the bonus token) raises
 * SV_ROW_EOS.  eos_id < 0 disables the rule; eos_id >= V is an argument
 * error.
 * Everything else is as for spec_verify_sample / spec_verify_greedy; the
 * workspace is spec_verify_workspace_size(B, gamma_max, V, dt, prm). */
sv_status spec_verify_sample_ragged(const void* target_logits, sv_dtype dt, const float* draft_probs,
                                    const int32_t* draft_ids, const int32_t* cu_draft, int32_t n_draft,
                                    const float* u_accept, const float* u_resample, int32_t B, int32_t gamma_max,
                                    int32_t V, sv_sampling_params prm, int32_t eos_id, int32_t* out_tokens,
                                    int32_t* out_num_accepted, uint32_t* out_row_flags, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* spec_verify_sample_ragged with q formed from the draft's logits (as in
 * spec_verify_sample_draft_logits): draft_logits [n_draft, V] (draft_dt),
 * packed like draft_ids, one row per draft position.  Workspace:
 * spec_verify_draft_logits_workspace_size(B, gamma_max, V, dt, draft_dt, prm). */
sv_status spec_verify_sample_ragged_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                                sv_dtype draft_dt, const int32_t* draft_ids, const int32_t* cu_draft,
                                                int32_t n_draft, const float* u_accept, const float* u_resample,
                                                int32_t B, int32_t gamma_max, int32_t V, sv_sampling_params prm,
                                                int32_t eos_id, int32_t* out_tokens, int32_t* out_num_accepted,
                                                uint32_t* out_row_flags, void* workspace, size_t workspace_bytes,
                                                void* stream);

sv_status spec_verify_greedy_ragged(const void* target_logits, sv_dtype dt, const int32_t* draft_ids,
                                    const int32_t* cu_draft, int32_t n_draft, int32_t B, int32_t gamma_max,
                                    int32_t V, int32_t eos_id, int32_t* out_tokens, int32_t* out_num_accepted,
                                    uint32_t* out_row_flags, void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify_sample_stats with q formed from the draft's logits: the
 * outputs of spec_verify_sample_draft_logits and spec_accept_stats_draft_logits
 * from one pass over the draft's and one over the target's logits.
 * Workspace: spec_verify_draft_logits_workspace_size. */
sv_status spec_verify_sample_stats_draft_logits(const void* target_logits, sv_dtype dt, const void* draft_logits,
                                               sv_dtype draft_dt, const int32_t* draft_ids, const float* u_accept,
                                               const float* u_resample, int32_t B, int32_t gamma, int32_t V,
                                               sv_sampling_params prm, int32_t* out_tokens, int32_t* out_num_accepted,
                                               uint32_t* out_row_flags, float* out_alpha, float* out_z_pq,
                                               float* out_z_qp, float* out_accept_prob, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* Kernel stages of a call, for the profiling hook below. */
typedef enum SV_ENUM_INT {
  SV_STAGE_ROWPASS = 0,       /* the streaming pass over the target logits (not the draft rows') */
  SV_STAGE_ROWFINAL = 1,      /* the target rows' finisher (kept sets, normalisers, draft gather) */
  SV_STAGE_ACCEPT = 2,        /* the acceptance decision launch (with the draws it takes itself) */
  SV_STAGE_DRAW_PARTIAL = 3,  /* untruncated draws, long drafts: the chunk sums after the decision */
  SV_STAGE_DRAW_FINISH = 4,   /* untruncated draws: the walk and rescan launch */
  SV_STAGE_STATS_PASS = 5,    /* statistics: the pass over streamed rows (not the untruncated rows' S64 pass before it) */
  SV_STAGE_STATS_FINISH = 6,  /* statistics: the per-position finish */
  SV_STAGE_GREEDY = 7,        /* greedy decision */
  SV_STAGE_QSUM = 8,          /* statistics: a dense q's row sums for Z' (on the library's side stream) */
  SV_STAGE_STATS_ZQP = 9,     /* statistics: Z' of listed rows with a dense q, after the q sums */
  SV_STAGE_COUNT = 10
} sv_stage;

/* Profiling hook (for benchmarks; process-wide, not thread-safe).  When both
 * events are non-NULL, every later call attaches them to the dispatch of
 * its kernel of stage `stage` (an sv_stage) on the call's stream:
 * `start_event` takes the kernel's start time and `stop_event` its end
 * time.  Both are hipEvent_t handles owned by the caller.  Passing NULL for
 * either turns that stage's hook off.  A stage absent from a call leaves
 * its events untouched.  Nothing else changes.  Returns
 * SV_ERR_INVALID_ARG for an unknown stage. */
sv_status spec_set_stage_timer(int32_t stage, void* start_event, void* stop_event);

/* spec_set_stage_timer(SV_STAGE_ROWPASS, start_event, stop_event). */
sv_status spec_set_rowpass_timer(void* start_event, void* stop_event);

/* Static description of a status code. */
const char* spec_status_string(sv_status status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
