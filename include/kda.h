/* libkda -- Kimi Delta Attention (KDA) forward operator for AMD MI355X (gfx950).
 *
 * The operator (Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (1)): for every sequence n and
 * head h independently, with state S in R^{dk x dv} entering as S0[n, h] (or zero),
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *
 * where g_t is the per-key-channel natural-log decay, expected in [g_min, 0] with g_min = -5
 * (§2.1.1, eq. (5)), and beta_t in [0, 1] is the delta-rule write strength.  The decay acts before
 * the delta update and o_t reads the state after token t's update.  q is multiplied by `scale`.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library allocates no
 *    device memory and keeps no pointer after the call's work has run on `stream`.  (The one
 *    fixed array it owns, behind kda_chunk_fwd_cp_noalloc, is part of its code object.)
 *  - Dense row-major layouts, token-major with heads interleaved ("B, T, H, d"):
 *      q, k  [B, T, H, dk]     v, o  [B, T, H, dv]     g [B, T, H, dk] (float32)
 *      beta  [B, T, H]         S0, S_T [N, H, dk, dv] (float32)
 *    q, k, v and beta share `in_dtype`; o has `out_dtype`.
 *  - Every pointer must be 16-byte aligned (beta: 4-byte aligned is enough).
 *  - Outputs (o, y, S_T, checkpoints, workspace, and a state updated in place) may overlap no
 *    input and no other output; read-only inputs may alias one another.  The one exception is
 *    S_T aliasing S0 exactly in an unsegmented prefill.  Any other overlap returns
 *    KDA_ERR_INVALID_ARGUMENT.
 *  - Work runs on the calling thread's current HIP device and is enqueued asynchronously on
 *    `stream` (0 = the null stream), which must belong to that device; nothing synchronises the
 *    host.  All argument checks run on the host before any launch: on error nothing is enqueued.
 *  - Results are deterministic: no atomics, fixed reduction orders.
 *  - Thread-safe and re-entrant.  The only process-wide state is a per-device record of which
 *    prefill kernels have had their LDS limit raised (set once, idempotent), the flag of the
 *    optional domain check below (used under a lock) and the per-device address of the fixed
 *    array of kda_chunk_fwd_cp_noalloc (looked up once, under a lock; the array's contents are
 *    shared by that entry point's calls, see there); error text is per thread.
 *  - Domain check (a debug aid, off by default): with the environment variable KDA_CHECK_RANGE=1,
 *    every entry point that reads g first checks on `stream` that each value lies in [-5, 0]
 *    (eq. (5) and the bound after it; NaN fails), synchronises `stream` to read the result, and
 *    returns KDA_ERR_RANGE without launching anything else if one does not.  The prefill kernel
 *    relies on this domain for the bf16 range of its rescale factors; outside it results are
 *    undefined (never an out-of-bounds access).  With the same variable, every entry point that
 *    takes cu_seqlens first checks on `stream` that the offsets run from 0 to T without
 *    decreasing, and returns KDA_ERR_INVALID_ARGUMENT if they do not.
 */
#ifndef LIBKDA_KDA_H
#define LIBKDA_KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size, aliasing, bad dtype   */
    KDA_ERR_UNSUPPORTED = 2,      /* a valid request the library does not implement (e.g. dk=96) */
    KDA_ERR_RANGE = 3,            /* g outside [-5, 0] (only with KDA_CHECK_RANGE=1, see below)  */
    KDA_ERR_HIP = 4               /* the HIP runtime reported an error (launch, no device)      */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* Chunkwise prefill (§2.1.1, eqs. (3)-(4): recurrent across chunks, parallel inside a chunk).
 *
 * Sequences: without `cu_seqlens` (NULL), N = B and row b of every [B, T, ...] tensor is one
 * sequence of T tokens.  With `cu_seqlens` (device int32 [N + 1], non-decreasing, cu[0] = 0,
 * cu[N] = T), B must be 1 and sequence n is tokens [cu[n], cu[n+1]) of the packed row; lengths
 * may be 0 (then S_T[n] = S0[n] and no output row belongs to it).  Out-of-range cu_seqlens
 * values are clamped inside the kernel (never an out-of-bounds access) but give meaningless
 * results.
 *
 * S0 may be NULL (zero entering state).  S_T may be NULL (final state not wanted) and may alias
 * S0 exactly (in-place state advance).  o and S_T must not overlap any input (cu_seqlens
 * included) or each other.
 *
 * Supported: dk in {64, 128}; dv in {64, 128}; in_dtype KDA_BF16 or KDA_F32; out_dtype KDA_BF16
 * or KDA_F32; T >= 0; B, H >= 1; N * H <= 2^30; H * max(dk, dv) <= 2^22 (KDA_ERR_UNSUPPORTED
 * beyond).
 *
 * Accuracy: relative L2 error of o and S_T against a float64 evaluation of eq. (1) on the same
 * stored inputs is about 2e-4 for random unit keys and stays below 5e-4 in the hardest regime
 * tested (beta = 1, weak decay, keys bunched around one direction); a bf16 o adds its own
 * rounding (1.66e-3 relative).  q and k are expected to be L2-normalised as eq. (2) produces them
 * (|q|, |k| <= 1 per entry): the kernel carries decayed q and k as float16.  v and S0 may have any
 * finite magnitude: the value path is rescaled by powers of two inside the kernel.
 *
 * Splitting in time (the in-device context parallelism of §5.1.1, on the decomposition of
 * §5.1.2, eq. (17); see kda_chunk_fwd_cp): with a workspace of at least
 * kda_chunk_fwd_workspace_size(N, B * T, H, dk, dv, cu_seqlens != NULL) bytes (16-byte aligned,
 * caller-owned, overlapping no input or output), the call plans by itself whether and how to
 * split sequences in time, on the device (no host synchronisation): a probe reads g over 8
 * chunks of 32 tokens spread evenly over the batch, then one planning workgroup reads the
 * sequence lengths (cu_seqlens, or the rows of a fixed-length batch), chooses a layout and a
 * segment length and writes the plan into the workspace.  Each sequence is cut by its own
 * length: longer sequences get more segments, those no longer than the segment length stay whole
 * and run beside the first pass.  A segment's transition M (eq. (17): its state is M S_in + S~)
 * vanishes once every entry is below 2^-140 of the identity it starts from; from there on its
 * outputs no longer depend on the state it is entered with.  Layouts: eager, where pass 1 runs
 * every segment with its outputs (the later ones entered with 0) and pass 2 runs each later
 * segment again from its true entering state only over the chunks before its transition
 * vanished; deferred, where the last segment is left to pass 2, which runs it whole.  From the
 * weakest decay per chunk the probe saw, the planner estimates the chunks a transition needs to
 * vanish, prices each candidate segment length in both layouts with a model of the two passes on
 * this GPU's compute units (a pass lasts at least its longest workgroup and at least its total
 * work over the units) and splits only when the best is expected to beat the whole-sequence
 * schedule by 5 % and to take at most 1.5 times it should no transition vanish.  Batches
 * with more than 16 whole-sequence workgroups (n_seq H dv / 64) per compute unit run whole.
 * Results agree with the whole-sequence run within the operator's tolerance (not bit for bit);
 * the plan, and with it the result, is a deterministic function of the inputs.  With workspace
 * NULL or too small, or S_T
 * aliasing S0, every sequence runs whole (workspace_bytes is then not checked).
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                         kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                         void* o, float* S_T, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of workspace kda_chunk_fwd needs to plan a split in time for n_seq sequences holding
 * total_tokens tokens in all, on the current device (the plan depends on its compute units):
 * packed = 0 for fixed-length rows (n_seq rows of total_tokens / n_seq tokens; 0 when no split
 * can pay), packed = 1 for cu_seqlens batches.  Either is an upper bound for what the plan uses:
 * the plan, 4 + 7 n_seq + 4 Smax + 64 int32 rounded up to 256 bytes, then Smax = min(n_seq (Pmax
 * - 1), total_tokens / Lmin) summaries of H x dk x (dv + dk) float32 and their H x dk / 64 int32
 * stop counts, with Pmax = min(16, ceil(2 CUs / (H dv / 64))) segments per sequence and Lmin =
 * max(1024, ceil(total_tokens / 64) rounded up to 32) tokens per segment; 0 beyond 65536
 * sequences and when the whole-sequence grid, n_seq H dv / 64 workgroups, exceeds 16 per
 * compute unit: such batches run whole.  0 for unsupported sizes. */
size_t kda_chunk_fwd_workspace_size(int32_t n_seq, int64_t total_tokens, int32_t H, int32_t dk,
                                    int32_t dv, int32_t packed);

/* kda_chunk_fwd that also emits prefix states (§5.4.1: the recurrent state of a prefix is what a
 * prefix cache stores and reuses; a chunkwise prefill already holds it at chunk ends).
 *
 * Same arguments and results as kda_chunk_fwd, plus: after every `ckpt_interval` tokens of a
 * sequence (a positive multiple of 32, the chunk length), the state after those tokens is written
 * to ckpt[n, h, j] for the j-th interval end (j = 0, 1, ...), as long as j < ckpt_capacity.
 * Layout: ckpt [N, H, ckpt_capacity, dk, dv] float32, caller-owned, 16-byte aligned.  Only whole
 * intervals are emitted: a sequence of length L yields min(floor(L / ckpt_interval),
 * ckpt_capacity) states (the last one equals S_T when L is a multiple of the interval); slots past
 * that are left untouched.  ckpt must not overlap an input, o or S_T.  ckpt_capacity = 0 (ckpt may then
 * be NULL) behaves exactly as kda_chunk_fwd.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED (interval not a positive multiple
 * of 32, or an unsupported shape) or KDA_ERR_HIP. */
kda_status kda_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* g,
                              const void* beta, const float* S0, const int32_t* cu_seqlens,
                              int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                              kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                              float* S_T, int32_t ckpt_interval, int32_t ckpt_capacity, float* ckpt,
                              hipStream_t stream);

/* kda_chunk_fwd with the decay computed inside the kernel from its logits by the bounded map of
 * §2.1.1, eq. (5):
 *
 *     g[b, t, h, c] = g_min * Sigmoid(exp(A_log[h]) * z[b, t, h, c]),   g_min = -5,
 *
 * so g never goes through memory (z is read in in_dtype, 2 bytes per channel for bf16, instead
 * of float32 g).  A_log is the per-head log-scale A_h of eq. (5).
 *
 * z: [B, T, H, dk] in in_dtype, 16-byte aligned; A_log: device float32 [H], 4-byte aligned.  Every
 * other argument, the layouts and the results are those of kda_chunk_fwd evaluated on that g
 * (the map runs in float32), the workspace and the split in time it enables included (its decay
 * probe maps the logits it samples the same way; kda_chunk_fwd_workspace_size gives the size).
 * o must not overlap z or A_log either.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT (also: z or A_log NULL or misaligned),
 * KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_chunk_fwd_gate(const void* q, const void* k, const void* v, const void* z,
                              const float* A_log, const void* beta, const float* S0,
                              const int32_t* cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t N,
                              int32_t dk, int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, void* o, float* S_T, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace kda_chunk_fwd_cp needs: N * (segments - 1) * H * (dk * (dv + dk) + dk / 64)
 * * 4 (the summaries and stop counts below), 0 when segments <= 1 or a size is not positive,
 * SIZE_MAX when the product does not fit in size_t. */
size_t kda_chunk_fwd_cp_workspace_size(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                       int32_t segments);

/* The segment count for kda_chunk_fwd_cp that suits a GPU with `slots` concurrent prefill
 * workgroups (one per CU: 256 on MI355X): the largest P <= 64 whose pass-1 value workgroups,
 * N*H*P*dv/64, fit in one round (its transition workgroups stop within a few chunks where the
 * keys' channels decay); 1 when P = 2 does not fit (then kda_chunk_fwd is as fast).  Host
 * arithmetic only (no device call); 1 for non-positive arguments. */
int32_t kda_chunk_fwd_cp_segments(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t slots);

/* kda_chunk_fwd with each sequence split in time into `segments` pieces that run in parallel:
 * the in-device context parallelism of §5.1.1 for long prefill with few heads, built on the
 * decomposition of §5.1.2, eq. (17): the state after a segment is M S_in + S~, with M the product
 * of the segment's per-token transitions (I - beta k k^T) Diag(exp(g)) and S~ the segment's state
 * when entered with zero.  For few, long sequences (N * H small) this puts more of the GPU to
 * work: one pass of T / segments tokens instead of one of T, plus a short second pass.
 *
 * Segment length: each sequence's own ceil(len / segments) rounded up to a multiple of 32 (pieces
 * past its end are empty).
 * Pass 1 runs every segment of every sequence and head with its outputs, the first entered with
 * S0 and the others with 0, and writes [S~ | M] (dk x (dv + dk), float32) for all but the last
 * to `workspace`, with, for every segment after the first, the number of its chunks before its
 * transition M vanishes (every entry zero, or below 2^-140 of the identity it starts from).
 * The workgroups of the transition columns stop at that point and store M as +0.0, which changes
 * no result by more than 2^-140 relative to the state carried in.  Pass 2 rebuilds the entering
 * state of each later segment, S_in(j) = M_{j-1} S_in(j-1) + S~_{j-1} (from the last earlier
 * segment whose M vanished), and runs the segment again over those chunks, whose outputs depend
 * on S_in(j) (all of them, and S_T for the last, where the transition never vanishes); the
 * outputs after them are those of pass 1, since there the state M S_in + S~ is S~ to that
 * precision.  Same results as kda_chunk_fwd within the operator's
 * tolerance (the summaries are computed with the same arithmetic; the combination uses split
 * bf16 products with float32 accumulation).
 *
 * N * H * segments <= 2^28 (KDA_ERR_UNSUPPORTED beyond).
 * workspace: device memory of at least kda_chunk_fwd_cp_workspace_size(N, H, dk, dv, segments)
 * bytes, 16-byte aligned, caller-owned, overlapping no input, o or S_T; ignored (may be NULL)
 * when segments == 1, which is exactly kda_chunk_fwd.  With segments > 1, S_T may not alias S0
 * (the first segment reads S0 while the last one writes S_T, in the same launch).  Other
 * arguments as kda_chunk_fwd.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT (also: segments < 1, workspace too small, misaligned
 * or overlapping), KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_chunk_fwd_cp(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, const int32_t* cu_seqlens, int32_t B,
                            int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                            kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                            float* S_T, int32_t segments, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Bytes of the fixed device array behind kda_chunk_fwd_cp_noalloc (32 MiB). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* kda_chunk_fwd_cp for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and results
 * bit for bit, with the segment summaries kept in a fixed array of KDA_NOALLOC_SCRATCH_BYTES that
 * each device's copy of the library holds from its first use there until the process ends.  The
 * call allocates nothing (no hipMalloc, no hipFree); the caller still passes inputs and outputs.
 * The array is written by pass 1 before pass 2 reads it, so nothing needs clearing between calls.
 * All calls on one device share that device's array: calls that may overlap in time on one
 * device (different streams, or other host threads) race on it and must be serialised by the
 * caller.  kda_chunk_fwd_cp_workspace_size(N, H, dk, dv, segments) must not exceed
 * KDA_NOALLOC_SCRATCH_BYTES (KDA_ERR_UNSUPPORTED otherwise, checked before anything runs).
 * Other arguments, checks and results as kda_chunk_fwd_cp. */
kda_status kda_chunk_fwd_cp_noalloc(const void* q, const void* k, const void* v, const float* g,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk,
                                    int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                                    void* o, float* S_T, int32_t segments, hipStream_t stream);

/* One decode token per (sequence, head), state updated IN PLACE (§5.4.2: at decode the state is
 * advanced in place every step and its traffic dominates).  eq. (1) with T = 1:
 *
 *     S <- Diag(exp(g)) S;  u = beta (v - S^T k);  S <- S + k u^T;  o = S^T (scale q).
 *
 * Layouts: q, k, g [N, H, dk]; v, o [N, H, dv]; beta [N, H]; S [N, H, dk, dv] float32.
 * Neither S nor o may overlap an input, nor each other.  Supported: dk, dv in {64, 128}.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const void* beta, float* S, int32_t N, int32_t H, int32_t dk,
                              int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                              void* o, hipStream_t stream);

/* kda_recurrent_step with the decay computed from its logits, g = g_min Sigmoid(exp(A_log[h]) z)
 * with g_min = -5 (§2.1.1, eq. (5)), as in kda_chunk_fwd_gate.  z: [N, H, dk] in in_dtype,
 * 16-byte aligned; A_log: device float32 [H].  Other arguments as kda_recurrent_step.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_recurrent_step_gate(const void* q, const void* k, const void* v, const void* z,
                                   const float* A_log, const void* beta, float* S, int32_t N,
                                   int32_t H, int32_t dk, int32_t dv, kda_dtype in_dtype,
                                   kda_dtype out_dtype, float scale, void* o, hipStream_t stream);

/* K decode tokens per (sequence, head) with one pass over the state: the decode-side variant
 * §5.4.2 describes for speculative decoding, where K drafted tokens are verified together and
 * the accepted ones are then replayed from their cached projected inputs.  The state is read
 * once, advanced through tokens 0..K-1 in registers (eq. (1) per token), and written back IN
 * PLACE after the first n_commit[n] tokens of sequence n (n_commit NULL: all K; 0: the state is
 * left untouched, e.g. a verification pass).  o receives every token's output, computed from the
 * states after each token whether or not they are committed; o may be NULL (outputs not wanted,
 * e.g. a replay pass).  n_commit values are clamped to [0, K].
 *
 * Layouts: q, k, g [N, K, H, dk]; v, o [N, K, H, dv]; beta [N, K, H]; S [N, H, dk, dv] float32;
 * n_commit device int32 [N] or NULL.  Neither S nor o may overlap an input (n_commit included),
 * nor each other.  Supported: dk, dv in {64, 128}.  K = 0 or N = 0 does nothing.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_recurrent_multi(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float* S, const int32_t* n_commit, int32_t N,
                               int32_t K, int32_t H, int32_t dk, int32_t dv, kda_dtype in_dtype,
                               kda_dtype out_dtype, float scale, void* o, hipStream_t stream);

/* kda_recurrent_multi fused with the steps the model applies around the operator (§2.1.1),
 * for serving and speculative decoding (§5.4.2: one kernel covers short convolution, input
 * norm, gating, the recurrence and the output norm, for the replayed and drafted tokens):
 *   before (eq. (2)): with conv_weight given, q, k and v are the projections before the short
 *     convolution and become Swish(ShortConv(.)) first, ShortConv being causal and depthwise per
 *     (head, channel):  x'_t = sum_{j < W} conv_weight[h, c, j] x_{t - W + 1 + j},  with the W - 1
 *     inputs before the first token taken from conv_state, Swish(x) = x Sigmoid(x);
 *     then q and k are L2-normalised per (token, head), x / max(||x||_2, 1e-12);
 *     beta = Sigmoid(beta_logit); g = -5 Sigmoid(exp(A_log[h]) z) (eq. (5));
 *   after (eq. (6) without W_o): y = Sigmoid(G) * RMSNorm(o~) per (token, head), with
 *     RMSNorm(o~) = o~ / sqrt(mean over dv of o~^2 + eps) * norm_weight.
 * The projections that produce q, k, v, z, beta_logit and G (and W_o after) need model weights
 * and stay with the caller.  State update, commit rule and o~ are those of kda_recurrent_multi;
 * the convolution window is committed with the state: conv_state receives, IN PLACE, the last
 * W - 1 inputs of each channel up to and including token n_commit[n] - 1 (0: untouched).
 *
 * Layouts: q, k, z [N, K, H, dk]; v, G, y [N, K, H, dv]; beta_logit [N, K, H], all in in_dtype;
 * A_log [H] float32; norm_weight [dv] float32, 16-byte aligned, or NULL (ones); eps >= 0;
 * conv_weight [H, 2 dk + dv, W] float32 (channels of q, then k, then v; tap W - 1 weights the
 * current token) or NULL (no convolution and no Swish: q, k, v are used as given);
 * conv_state [N, H, 2 dk + dv, W - 1] in in_dtype, oldest input first, 16-byte aligned (may be
 * NULL when W = 1);
 * conv_width W in [1, 4] (ignored without conv_weight); S [N, H, dk, dv] float32; n_commit device
 * int32 [N] or NULL.  y may be NULL (no outputs; G is then not read).  None of S, conv_state and y
 * may overlap an input or each other.  Supported: dk, dv in {64, 128}.
 * Returns KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP. */
kda_status kda_recurrent_multi_fused(const void* q, const void* k, const void* v, const void* z,
                                     const float* A_log, const void* beta_logit, const void* G,
                                     const float* norm_weight, float eps, const float* conv_weight,
                                     void* conv_state, int32_t conv_width, float* S,
                                     const int32_t* n_commit, int32_t N, int32_t K, int32_t H,
                                     int32_t dk, int32_t dv, kda_dtype in_dtype,
                                     kda_dtype out_dtype, float scale, void* y, hipStream_t stream);

/* Static description of a status code.  Never NULL. */
const char* kda_status_string(kda_status status);

/* Human-readable detail of the last error returned on the calling host thread ("" if none). */
const char* kda_last_error(void);

/* Library ABI version: (major << 16) | minor. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_KDA_H */
