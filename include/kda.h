/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * KDA is the gated delta-rule linear-attention layer.  Per sequence and head,
 * with a dk x dv state S and tokens t in order:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,        alpha_t = exp(g_t) per key channel
 *
 *   ("Kimi K3.1 Pro 架构完全拆解", §3.1 single-head recurrence; §3.2 for
 *    the bounded log-decay g in (-5, 0) and alpha = exp(g).)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every buffer is a caller-owned DEVICE pointer unless its name ends in
 *   _host.  The library allocates no device memory; it keeps no pointer after
 *   a call returns, except a small pool of pinned host staging buffers it
 *   uses to upload its own schedule (freed at process exit).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call validates its arguments on the host first; on failure it
 *   returns a negative status and enqueues nothing.  On success the work is
 *   enqueued asynchronously on `stream`; no call synchronises.
 * - HIP graph capture: the prefill calls and kda_segment_transition upload
 *   their schedule from a pinned host buffer that later calls reuse, so a
 *   captured copy would read stale tables on replay; on a stream that is
 *   capturing they return KDA_ERR_UNSUPPORTED and enqueue nothing.  The
 *   decode calls (step and replay, plain and gated) and kda_segment_scan
 *   upload nothing and launch one kernel each; they may be captured.
 * - dk = dv = 128 and the chunk length C = 64 are fixed in this version of the library.
 * - Element type of q, k, v, g, beta and o is `dt`: KDA_F32 (fp32) or
 *   KDA_BF16 (bfloat16).  States, M and S~ are always fp32.  All arithmetic
 *   accumulates in fp32; with KDA_BF16 the matrix products take bf16
 *   operands, with KDA_F32 fp32 operands.
 * - Layouts are row-major, last index fastest:
 *       q, k, g : [T_total, H, dk]     v, o : [T_total, H, dv]
 *       beta    : [T_total, H]         states : [num_seqs, H, dk, dv]
 *   A batch of B fixed-length sequences of length T is the packed layout
 *   with cu_seqlens = {0, T, 2T, ..., BT}.
 * - Every device pointer must be 16-byte aligned, except beta, which needs
 *   only the alignment of its element type (so [T, H] beta can be sliced by
 *   token).
 * - Preconditions NOT checked (results are unspecified if violated):
 *   g in [-5, 0] (the gate's bound that keeps every 16-token cumulative
 *   log-decay above -80, "Kimi K3.1 Pro 架构完全拆解" §3.2) and finite
 *   inputs.  q and k are
 *   used as given (the layer L2-normalises them before this call); no
 *   1/sqrt(dk) scale is applied.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kda_status;

#define KDA_OK 0
#define KDA_ERR_INVALID_ARG (-1) /* NULL required pointer, bad size, bad cu_seqlens, misaligned */
#define KDA_ERR_UNSUPPORTED (-2) /* dk/dv other than 128, unknown dtype, capturing stream */
#define KDA_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than the size query returned */
#define KDA_ERR_HIP (-4)         /* a HIP runtime call or launch failed; outputs undefined */

typedef int32_t kda_dtype;
#define KDA_F32 0
#define KDA_BF16 1

#define KDA_CHUNK 64
#define KDA_HEAD_DIM 128

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t kda_version(void);

/*
 * Planner query (host only, no HIP calls): how many segments the chunked
 * prefill of element type dt on the automatic path will cut sequence
 * `seq_len` into, for a batch whose total (sequence, head) count is
 * C = num_seqs * H.
 *   split_hint = 0 : automatic: split long sequences only when the unsplit
 *                    work would leave most compute units idle.  KDA_F32
 *                    (and KDA_BF16 outside the next case): C < 64 cuts into
 *                    min(64, chunks / 4) segments.  KDA_BF16 with
 *                    8 <= C <= 128: min(1 + 256 / C, chunks / 12) segments
 *                    when that is at least 3, else none (the fused
 *                    planner, each of its passes one workgroup per compute
 *                    unit);
 *   split_hint = 1 : never split;
 *   split_hint = n > 1 : cut every sequence longer than one chunk into
 *                    min(n, number of its chunks) chunk-aligned segments.
 * Returns >= 1 (or 1 for seq_len <= 0), or a negative status for bad input.
 * kda_plan_num_segments is the KDA_F32 answer.  The sequence-split planner
 * follows "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度", §1.2 (intra-device,
 * SM-level context parallelism).
 */
int32_t kda_plan_num_segments_dt(int64_t seq_len, int32_t num_seqs, int32_t H,
                                 int32_t split_hint, kda_dtype dt);
int32_t kda_plan_num_segments(int64_t seq_len, int32_t num_seqs, int32_t H, int32_t split_hint);

/*
 * Chunked prefill over packed variable-length sequences.
 *
 * Computes, for each sequence n (tokens [cu[n], cu[n+1])) and head h, the
 * recurrence above from S_0 = initial_state[n,h] (or zero), writes o for
 * every token and, if final_state != NULL, the state after the last token.
 * It uses the chunkwise form ("Kimi K3 的架構" (hao.cnyes.com), §六 FlashKDA
 * 演算法): a chunk-prep step per (chunk, head) builds the decayed operands,
 * L = StrictTril(Diag(beta) K_decay K_inv^T), INV = (I + L)^-1 and
 * M_qk = tril(Q_decay K_inv^T); a state-carrying step per (sequence, head)
 * walks the chunks in order:
 *     U = INV Diag(beta)(V - K_decay S);  O = Q_decay S + M_qk U;
 *     S = Diag(a_last) S + K_restore^T U.
 * Chunks restart at every sequence start; a sequence's last chunk may be
 * shorter than 64 tokens.  Long sequences may be cut into segments whose
 * transition pairs are combined by a prefix scan and then replayed (see
 * kda_plan_num_segments and kda_segment_transition); the result is the same
 * up to fp32 rounding.
 * Two implementations compute the same result.  With KDA_BF16, a fused
 * kernel builds each chunk's operands on chip while it carries the state
 * (the workspace then holds no per-chunk operands): without a split for at
 * least 129 (sequence, head) pairs; with the bf16 automatic cut (8 to 128
 * pairs, kda_plan_num_segments_dt) or an explicit split into at least 256
 * (segment, head) pairs, in the planner's segment pass and replay.
 * Otherwise a chunk-parallel prep kernel writes the per-chunk operands to
 * the workspace and a state-carrying kernel reads them.
 * kda_chunk_prefill_ex chooses between them explicitly.
 *
 *   num_seqs         : N >= 0 sequences.
 *   cu_seqlens_host  : HOST, N+1 int64, cu[0] = 0, nondecreasing.  The
 *                      library derives its schedule from it and uploads that
 *                      schedule into `workspace` with an async copy.
 *   H, dk, dv, dt    : heads (>= 1), 128, 128, element type.
 *   q, k, v, g, beta : inputs (layouts above); g is a natural-log decay.
 *   initial_state    : [N, H, dk, dv] fp32, or NULL for zeros.
 *   o                : [T_total, H, dv] output of type dt.
 *   final_state      : [N, H, dk, dv] fp32 output, or NULL (not written).
 *                      final_state == initial_state is allowed (in-place
 *                      resume); any other overlap between outputs and
 *                      inputs is not.
 *   split_hint       : as in kda_plan_num_segments.
 *   workspace        : DEVICE scratch of at least the queried size, 256-byte
 *                      aligned; contents are undefined after the call.
 * A length-0 sequence writes its initial state (or zeros) to final_state.
 */
size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                        int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                        int32_t split_hint);

kda_status kda_chunk_prefill(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                             int32_t dk, int32_t dv,
                             kda_dtype dt, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *initial_state,
                             void *o, float *final_state, int32_t split_hint, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * The prefill with every option in one call: which implementation runs, the
 * state checkpoints of kda_chunk_prefill_ckpt / kda_chunk_prefill_ckpt_all
 * and the layer steps of kda_chunk_prefill_gated (the paragraphs of those
 * calls define them; any combination is allowed).  The calls above are this
 * one with some options fixed.
 *
 *   path          : KDA_PATH_AUTO (the library chooses as described for
 *                   kda_chunk_prefill), KDA_PATH_TWO_KERNEL (chunk-prep
 *                   kernel, then the state-carrying kernel; any dtype and
 *                   split), or KDA_PATH_FUSED (the fused kernel; KDA_BF16
 *                   only; split_hint = 0 then means no split, and a split
 *                   (split_hint > 1) runs the planner's segment pass and
 *                   replay on it).
 *   ckpt_align    : 0 for no checkpoints; else the hash-block length, a
 *                   positive multiple of 64, with pos0_host and ckpt_state
 *                   as for kda_chunk_prefill_ckpt; ckpt_all = 1 writes every
 *                   aligned position (ckpt_state then as ckpt_states of
 *                   kda_chunk_prefill_ckpt_all), 0 the last one only.
 *   A_log, g_min, qk_norm_eps, out_gate, out_norm_weight, out_norm_eps :
 *                   as for kda_chunk_prefill_gated (A_log NULL: g is the log
 *                   decay; qk_norm_eps 0: q and k as given; out_gate NULL: o
 *                   as the recurrence gives it).
 * opts == NULL means path AUTO with no checkpoints and no layer steps.  The
 * workspace size depends on the path: query it with
 * kda_chunk_prefill_ex_workspace_size and the same options (it returns 0 for
 * an invalid or unsupported request).
 */
#define KDA_PATH_AUTO 0
#define KDA_PATH_TWO_KERNEL 1
#define KDA_PATH_FUSED 2

typedef struct kda_prefill_options {
  int32_t path;
  int32_t ckpt_align;
  int32_t ckpt_all;
  float g_min;
  float qk_norm_eps;
  float out_norm_eps;
  const int64_t *pos0_host;
  float *ckpt_state;
  const float *A_log;
  const void *out_gate;
  const float *out_norm_weight;
} kda_prefill_options;

size_t kda_chunk_prefill_ex_workspace_size(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                           int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                           int32_t split_hint, const kda_prefill_options *opts);

kda_status kda_chunk_prefill_ex(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                const void *k, const void *v, const void *g, const void *beta,
                                const float *initial_state, void *o, float *final_state,
                                int32_t split_hint, const kda_prefill_options *opts,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory (code in
 * tight serving loops, or harnesses that forbid hipMalloc): it takes no
 * workspace and allocates nothing.  It runs the fused kernel (KDA_BF16 only,
 * no planner split) with its schedule tables in a fixed device array of
 * KDA_NOALLOC_SCRATCH_BYTES that each device the library runs on holds until
 * the process ends; the tables are uploaded with a host-to-device copy from
 * a fixed host buffer.
 *   Returns KDA_ERR_UNSUPPORTED for dt != KDA_BF16 or dk, dv != 128, and
 *   KDA_ERR_WORKSPACE when the schedule exceeds the array (40 bytes per
 *   sequence plus alignment: about 26,000 sequences).
 * Every call on one device uses that device's array, which keeps the last
 * call's contents: calls that overlap on one GPU (on different streams, or
 * from different host threads without ordering) race.  Arguments and results
 * are otherwise those of kda_chunk_prefill with split_hint = 0.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (1 << 20)

kda_status kda_chunk_prefill_noalloc(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                     int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                     const void *k, const void *v, const void *g,
                                     const void *beta, const float *initial_state, void *o,
                                     float *final_state, void *stream);

/*
 * kda_chunk_prefill that also writes, per sequence, the state at its last
 * hash-aligned position: the KDA checkpoint a prefix cache keeps after each
 * forward pass ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §三 3.2, the KDA
 * kernel persists the state at the last hash-aligned position it processed;
 * "Kimi K3.1 Pro 架构完全拆解" §8.2, checkpoints only on hash-block ends).
 *
 *   pos0_host  : HOST [num_seqs], the absolute position of each sequence's
 *                first token (a resumed prefill starts past 0), each a
 *                non-negative multiple of 64; NULL means all 0.
 *   ckpt_align : the hash-block length in tokens, a positive multiple of 64
 *                (for example 512).
 *   ckpt_state : [num_seqs, H, dk, dv] fp32.  For sequence n of length L the
 *                checkpoint position is p = floor((pos0 + L) / ckpt_align)
 *                * ckpt_align; when p > pos0, slice n receives the state after
 *                the sequence's first p - pos0 tokens (its initial state
 *                included; equal to its final state when p = pos0 + L).
 *                Otherwise slice n is not written.
 * Everything else, the workspace size included, is as for kda_chunk_prefill.
 */
kda_status kda_chunk_prefill_ckpt(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                  int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                  const void *k, const void *v, const void *g, const void *beta,
                                  const float *initial_state, void *o, float *final_state,
                                  int32_t split_hint, const int64_t *pos0_host,
                                  int32_t ckpt_align, float *ckpt_state, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prefill_ckpt, but with a checkpoint at every hash-aligned
 * position rather than the last one only: the optional form of the KDA
 * kernel's state persistence ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度"
 * §三 3.2, a state per hash block boundary; "Kimi K3.1 Pro 架构完全拆解"
 * §8.2).  For sequence n the positions are p = m * ckpt_align with
 * pos0[n] < p <= pos0[n] + L_n, in increasing order; the k-th of them gets
 * the state after the sequence's first p - pos0[n] tokens.
 *
 *   ckpt_states : [kda_prefill_num_checkpoints(...), H, dk, dv] fp32, the
 *                 sequences' checkpoints one after another (sequence 0's
 *                 first); may be NULL when there are none.
 * pos0_host and ckpt_align as for kda_chunk_prefill_ckpt; everything else,
 * the workspace size included, as for kda_chunk_prefill.
 */
kda_status kda_chunk_prefill_ckpt_all(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                      int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                      const void *q, const void *k, const void *v,
                                      const void *g, const void *beta,
                                      const float *initial_state, void *o, float *final_state,
                                      int32_t split_hint, const int64_t *pos0_host,
                                      int32_t ckpt_align, float *ckpt_states, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * The number of checkpoints kda_chunk_prefill_ckpt_all writes: the
 * ckpt_align-aligned positions p with pos0[n] < p <= pos0[n] + L_n, summed
 * over the sequences (host only).  -1 for invalid arguments (cu_seqlens not
 * starting at 0 or decreasing, pos0 negative or not a multiple of 64,
 * ckpt_align not a positive multiple of 64).
 */
int64_t kda_prefill_num_checkpoints(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                    const int64_t *pos0_host, int32_t ckpt_align);

/*
 * kda_chunk_prefill with the layer's steps on either side of the recurrence
 * fused into its kernels, so that none of them costs a pass over [T, H, d]:
 *
 *   before ("Kimi K3.1 Pro 架构完全拆解" §3.2; "Kimi K3 的架構" §七)
 *     A_log != NULL : g holds the raw gate logits z, and the log decay is
 *                     g_min * sigmoid(exp(A_log[h]) * z), in (g_min, 0).
 *                     A_log: DEVICE [H] fp32, the per-head log scale;
 *                     g_min: -5 <= g_min < 0 (the pages fix -5).
 *                     A_log == NULL: g is the log decay, g_min is ignored.
 *     qk_norm_eps > 0 : each (token, head) row of q and of k is divided by
 *                     sqrt(sum of its squares + qk_norm_eps) first;
 *                     qk_norm_eps == 0: q and k are used as given.
 *   after ("Kimi K3.1 Pro 架构完全拆解" §3.3)
 *     out_gate != NULL : each (token, head) row of the output over its dv
 *                     channels is replaced by
 *                       sigmoid(out_gate) * w * o / sqrt(mean(o^2) + out_norm_eps)
 *                     out_gate: [T_total, H, dv] of type dt, the logits of
 *                     the full-rank output gate (its projection is not
 *                     done here), must not overlap o; out_norm_weight: DEVICE
 *                     [dv] fp32 (w), or NULL for ones; out_norm_eps > 0.
 *                     out_gate == NULL: o is the recurrence output.
 *
 * final_state is the state of the recurrence (it is not normalized).
 * Everything else, the workspace size included, is as for kda_chunk_prefill.
 * Invalid values (g_min outside [-5, 0), a negative or non-finite
 * qk_norm_eps, out_norm_eps <= 0 with a gate, misaligned pointers) return
 * KDA_ERR_INVALID_ARG before anything is enqueued.
 */
kda_status kda_chunk_prefill_gated(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                   const void *k, const void *v, const void *g, const void *beta,
                                   const float *A_log, float g_min, float qk_norm_eps,
                                   const void *out_gate, const float *out_norm_weight,
                                   float out_norm_eps, const float *initial_state, void *o,
                                   float *final_state, int32_t split_hint, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * One decode step for N independent sequences, updating the state IN PLACE
 * ("Kimi K3 的架構" (hao.cnyes.com), §六, the alternative form the decode
 * kernel follows; "Kimi K3.1 Pro 架构完全拆解" §3.4, state updated in place):
 *     DS = Diag(exp(g)) S;  u = beta (v - DS^T k);  S = DS + k u^T;
 *     o = S^T q  (= DS^T q + (k . q) u)
 *
 *   q, k, g : [N, H, dk] of type dt;  v : [N, H, dv];  beta : [N, H].
 *   state   : [N, H, dk, dv] fp32, read and overwritten.
 *   o       : [N, H, dv] of type dt; must not overlap any input or state.
 * N = 0 is a no-op.
 */
kda_status kda_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                           const void *q, const void *k, const void *v, const void *g,
                           const void *beta, float *state, void *o, void *stream);

/*
 * kda_decode_step with the layer's steps fused in ("Kimi K3.1 Pro 架构完全拆解"
 * §3.4: the decode kernel also does the input normalization, the gating and
 * the output norm; §3.2, §3.3 for the steps): A_log, g_min, qk_norm_eps,
 * out_gate ([N, H, dv] of type dt), out_norm_weight and out_norm_eps mean
 * what they mean for kda_chunk_prefill_gated.  The state stays the
 * recurrence's.
 */
kda_status kda_decode_step_gated(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                 const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const float *A_log, float g_min,
                                 float qk_norm_eps, const void *out_gate,
                                 const float *out_norm_weight, float out_norm_eps,
                                 float *state, void *o, void *stream);

/*
 * Speculative-decode replay for N sequences ("Kimi K3.1 Pro 架构完全拆解"
 * §3.4; "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §四): the state is not
 * rolled back from a snapshot but rebuilt from the cached projected inputs
 * of the accepted draft tokens.  Per sequence n, from `state` (the state
 * before the draft window), the decode step above runs over the first
 * m_n = clamp(accepted[n], 0, W) cached tokens (their outputs are not
 * produced), then over the P new tokens: the bonus token first, then the
 * next window's drafts.  The state after the accepted tokens and the bonus
 * token is written back (after the accepted tokens alone when P = 0); the
 * later drafts' states are not kept.
 *
 *   W        : cached window length, 0 <= W <= KDA_REPLAY_MAX_TOKENS.
 *   accepted : DEVICE int32 [N], accepted draft tokens per sequence (values
 *              outside [0, W] are clamped; read on the device, no sync).
 *   ck, cg   : [N, W, H, dk] of type dt;  cv : [N, W, H, dv];  cbeta : [N, W, H].
 *              May be NULL when W == 0.
 *   P        : new tokens, 0 <= P <= KDA_REPLAY_MAX_TOKENS.
 *   q, k, g  : [N, P, H, dk] of type dt;  v : [N, P, H, dv];  beta : [N, P, H].
 *              May be NULL when P == 0.
 *   state    : [N, H, dk, dv] fp32, read and overwritten.
 *   o        : [N, P, H, dv] of type dt: the new tokens' outputs; must not
 *              overlap any input or the state.  May be NULL when P == 0.
 * The state is read once and written once whatever W and P are.  N = 0 is a
 * no-op.  Validation failures return before anything is enqueued.
 */
#define KDA_REPLAY_MAX_TOKENS 64
kda_status kda_decode_replay(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                             int32_t W, const int32_t *accepted, const void *ck, const void *cv,
                             const void *cg, const void *cbeta, int32_t P, const void *q,
                             const void *k, const void *v, const void *g, const void *beta,
                             float *state, void *o, void *stream);

/*
 * kda_decode_replay with the layer's steps fused in (as
 * kda_decode_step_gated).  The gate and the q / k norms apply to the cached
 * tokens as to the new ones, so the window cache holds the raw inputs (with
 * A_log, cg holds gate logits like g); out_gate is [N, P, H, dv] of type dt,
 * the new tokens' output gate logits.
 */
kda_status kda_decode_replay_gated(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                   int32_t W, const int32_t *accepted, const void *ck,
                                   const void *cv, const void *cg, const void *cbeta, int32_t P,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *A_log, float g_min,
                                   float qk_norm_eps, const void *out_gate,
                                   const float *out_norm_weight, float out_norm_eps,
                                   float *state, void *o, void *stream);

/*
 * Segment transition pairs ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度", §二,
 * the KCP decomposition): for each packed segment s (tokens
 * [cu[s], cu[s+1])) and head h,
 *     M[s,h]       = M_T ... M_1,  M_r = (I - beta_r k_r k_r^T) Diag(exp(g_r))
 *     S_tilde[s,h] = the state after the segment when it starts from S = 0
 * so that the state after the segment from any entry state S_in is
 * S_tilde + M S_in, and pairs compose associatively:
 * (M2, S2) after (M1, S1) = (M2 M1, S2 + M2 S1).
 *
 *   cu_seglens_host : HOST, num_segs+1 int64, as cu_seqlens_host above.
 *   k, v, g, beta : as for kda_chunk_prefill (q is not needed).
 *   M       : [num_segs, H, dk, dk] fp32 output.
 *   S_tilde : [num_segs, H, dk, dv] fp32 output; must not overlap M.
 *   workspace : DEVICE scratch of at least the queried size.
 * A length-0 segment gives M = I and S_tilde = 0.
 */
size_t kda_segment_transition_workspace_size(int32_t num_segs,
                                             const int64_t *cu_seglens_host, int32_t H,
                                             int32_t dk, int32_t dv, kda_dtype dt);

kda_status kda_segment_transition(int32_t num_segs, const int64_t *cu_seglens_host,
                                  int32_t H, int32_t dk, int32_t dv, kda_dtype dt, const void *k, const void *v,
                                  const void *g, const void *beta, float *M, float *S_tilde,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefix scan of segment transition pairs ("部署 Kimi K3：从 KDA Kernel 到
 * Fleet 调度", §二: pairs compose associatively; in the cross-device KCP each
 * device folds the pairs of the shards before its own into its entry state).
 * For pairs (M_j, S_tilde_j), j = 0 .. num_segs-1, per head h:
 *     S_in[0] = initial_state (or zero),
 *     S_in[j+1] = S_tilde_j + M_j S_in[j],
 * so S_in[j] is the state entering segment j and S_in[num_segs] the state
 * after the last one.  With kda_segment_transition on each shard of a
 * sequence, this call, then kda_chunk_prefill of shard j from S_in[j], the
 * shards' outputs and states equal those of one prefill over the sequence.
 *
 *   M        : [num_segs, H, dk, dk] fp32, row-major, as kda_segment_transition
 *              writes it.
 *   S_tilde  : [num_segs, H, dk, dv] fp32.
 *   initial_state : [H, dk, dv] fp32, or NULL for zero.
 *   S_in     : [num_segs + 1, H, dk, dv] fp32 output; must not overlap M,
 *              S_tilde or initial_state (KDA_ERR_INVALID_ARG).
 * num_segs = 0 writes S_in[0] only.  Serial over the pairs, parallel over
 * heads and 16-column blocks, fp32 throughout (fp32 matrix cores).  No
 * workspace and no schedule upload: the call launches one kernel and may be
 * captured into a HIP graph.  H <= 2^24.
 */
kda_status kda_segment_scan(int32_t num_segs, int32_t H, int32_t dk, int32_t dv, const float *M,
                            const float *S_tilde, const float *initial_state, float *S_in,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
