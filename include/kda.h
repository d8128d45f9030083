/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked Kimi Delta Attention forward.
 *
 * Citation key:
 *   P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核"
 *        (guancyxx.cn), §一 (the gated delta-rule state update) and §二 2.1-2.4
 *        (chunk size 16, the token-parallel / chunk-recurrent split, the 16 x 16
 *        inverse, base-2 exponentials).
 *   P2 = FlashKDA README mirror (ai-feeds.com), section "内核 API" (Kernel API):
 *        the argument table of flash_kda.fwd and its four usage notes.
 *
 * What kda_fwd computes, for every sequence n and head h, with a K x V state S
 * per (n, h) kept in math layout S[k][v]:
 *   a_t[k] = lower_bound * sigmoid(exp(A_log[h]) * (g_t[k] + dt_bias[h][k]))
 *   beta_t = sigmoid(beta_t logit)
 *   kn_t   = k_t / sqrt(|k_t|^2 + 1e-6),  qn_t = scale * q_t / sqrt(|q_t|^2 + 1e-6)
 *   S      = diag(exp(a_t)) S;   S += beta_t kn_t (v_t - S^T kn_t)^T;   o_t = S^T qn_t
 * (P1 §一 gives a simplified scalar-gate form of this update; the per-channel
 * gate shape and the in-kernel gate / L2-norm / sigmoid activations come from
 * P2's argument table and its chunk_kda call.  The exact gate activation is not
 * printed on the pages: the bounded sigmoid form above is this library's
 * reading, chosen because it maps any raw gate into (lower_bound, 0).)
 *
 * All tensor pointers are DEVICE pointers to contiguous row-major buffers on
 * the current HIP device; q, k, g, v, out, dt_bias and the states must be
 * 16-byte aligned.  The caller owns every buffer, including the
 * workspace; the library never allocates or frees device memory.  kda_fwd only
 * enqueues work on `stream` (no host synchronisation, no device reads on the
 * host); buffers must stay alive until the stream has passed the call.  It
 * enqueues kernel launches only (no memsets or copies), so a call can be
 * captured into a HIP graph and replayed with the same buffers; so can
 * kda_fwd_ex without events or parts, kda_fwd_segmented and kda_decode.
 *
 * Shapes (P2 Kernel API), with N = B without cu_seqlens, len(cu_seqlens) - 1 with:
 *   q, k, g        bf16  [B, T, H, K]
 *   v              bf16  [B, T, H, V]
 *   beta           bf16  [B, T, H]          (logits; sigmoid applied inside)
 *   out            bf16  [B, T, H, V]       (written; rounded to nearest even)
 *   A_log          fp32  [H]
 *   dt_bias        fp32  [H, K]
 *   initial_state  bf16 | fp32 | none  [N, H, V, K]   (stored [n,h,v,k] = S[k][v])
 *   final_state    bf16 | fp32 | none  [N, H, V, K]   (written)
 *   cu_seqlens     int64 [N + 1] or NULL  (then B must be 1 and T is the total)
 * K = V = 128 is required (P2 Kernel API notes).
 *
 * Numerical range: the chunk recurrence multiplies fp16 operands with fp32
 * accumulation.  Values derived from v and the state (the state itself, the
 * per-chunk residuals) must stay below 65504 in magnitude; inputs drawn from
 * activations of O(1..1000) scale satisfy this with a wide margin.  Beyond
 * it an operand becomes infinite, the state of that (sequence, head) ends
 * non-finite, and the call reports KDA_STATUS_OVERFLOW in its status word.
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define KDA_OK 0
#define KDA_EINVAL 1       /* null required pointer, misaligned tensor, bad size, K or V != 128,
                              B != 1 with cu_seqlens, lower_bound outside [-5, 0], non-finite
                              scale */
#define KDA_EDTYPE 2       /* bad state dtype code, pointer/dtype mismatch, or initial and
                              final state dtypes differ (P2 Kernel API notes) */
#define KDA_EWORKSPACE 3   /* workspace too small (see kda_fwd_workspace_bytes) */
#define KDA_EUNSUPPORTED 4 /* current device is not gfx950 */
#define KDA_EHIP 5         /* a HIP runtime call or kernel launch failed */

/* State dtype codes. */
#define KDA_DTYPE_NONE 0
#define KDA_DTYPE_BF16 1
#define KDA_DTYPE_FP32 2

/* Device-side status word (kda_fwd_check_status): KDA_STATUS_OK, or an OR of
   these bits. */
#define KDA_STATUS_OK 0
#define KDA_STATUS_BAD_CU_SEQLENS 1 /* cu_seqlens[0] != 0, not monotone, or cu_seqlens[N] != T;
                                       then no token was processed and neither out nor
                                       final_state is written, on every path */
#define KDA_STATUS_SYNC_TIMEOUT 4   /* a wait between the waves of a recurrence or fused workgroup
                                       gave up (0.06 to 0.9 s without progress; not expected in
                                       operation): out and final_state are not meaningful */
#define KDA_STATUS_OVERFLOW 2       /* the chunk state of some (sequence, head) ended non-finite:
                                       a value outside the fp16 operand range (see "Numerical
                                       range" above) or a non-finite input; out and final_state
                                       of that pair are not meaningful */

/* Chunk size of the chunked form (P1 §二 2.1 uses 16). */
#define KDA_CHUNK 16

/* Execution paths (kda_fwd_ex).  Both compute the same chunked form; their
   results differ only in rounding.
   KDA_PATH_SPLIT: the two stages of P1 §二 2.2 as two kernels, the chunk
     records handed over through the workspace in HBM (16-, 32- or 64-token
     chunks, optional overlap of the stages by parts);
   KDA_PATH_FUSED: one kernel per (sequence, head, value tile) that builds each
     chunk's record in LDS a few chunks ahead of the recurrence that consumes
     it, so the records never reach HBM (16-token chunks, one part);
   KDA_PATH_AUTO: the library's choice.  On MI355X the fused kernel is
     faster for batches of many short sequences and the split path whenever
     a sequence is long.  With cu_seqlens the lengths are known only on the
     device, so both paths are enqueued and the scheduler kernel picks one
     from the chunk counts (the other path's kernels exit at once); for B
     sequences of T tokens the host applies the same estimate and enqueues
     only the path it picks.  The workspace is the split path's. */
#define KDA_PATH_AUTO 0
#define KDA_PATH_SPLIT 1
#define KDA_PATH_FUSED 2

/*
 * kda_fwd -- enqueue the chunked KDA forward pass on `stream`.
 *
 * The work is a scheduler kernel that turns cu_seqlens into per-sequence
 * tables and a longest-first work order, then the two stages of P1 §二 2.2:
 * chunk prep (gate activation, L2 norm, in-chunk decay, the L / Mqk matrices
 * and the 16 x 16 unit-lower-triangular inverse) and the chunk recurrence (the
 * chunk-by-chunk delta-rule state update and the output).  For B sequences
 * of T tokens on the split path the tables are a function of the chunk index:
 * no scheduler kernel runs, the prep kernel computes the entries and writes the
 * workspace header itself.  kda_fwd leaves the execution path to the library
 * (KDA_PATH_AUTO); kda_fwd_ex selects it.
 * Without cu_seqlens (B sequences of T tokens, lengths known on the host)
 * kda_fwd also cuts the sequences into segments (kda_fwd_segmented with
 * kda_fwd_segments' count) when that count is above 1 -- few heads and long
 * sequences, where one chain per (sequence, head) leaves the chip idle -- and
 * the workspace holds the segmented layout; kda_fwd_workspace_bytes sizes for
 * it.  With a smaller workspace the sequences run uncut.
 *
 * initial_state / final_state: NULL with dtype KDA_DTYPE_NONE, or a pointer
 * with KDA_DTYPE_BF16 / KDA_DTYPE_FP32.  When both are given their dtypes must
 * match.  A NULL initial state means a zero state; a NULL final state is not
 * written.  final_state == initial_state (the same buffer) is allowed; any
 * other overlap between inputs and outputs is undefined.
 * cu_seqlens: NULL, or num_seqs + 1 int64 prefix sums on the device (B == 1).
 * Its contents are checked on the device (see kda_fwd_check_status).
 * workspace: device memory, 256-byte aligned, of at least
 * kda_fwd_workspace_bytes_ex(B, T, H, num_seqs, cu != NULL, 0, 0, KDA_PATH_AUTO)
 * bytes (tables and the chunk records, about 864 B per token-head) --
 * kda_fwd_workspace_bytes gives a size that suits every path (and the
 * segmented form kda_fwd may take).  Its contents
 * are scratch between calls except for the status word.
 * stream: a hipStream_t (NULL = the default stream).
 *
 * With no tokens (B * T == 0) the token tensors q, k, v, g, beta and out are
 * empty and may be NULL; the final state is then the initial state.
 * Every argument error is detected on the host before any HIP call is made.
 * Returns KDA_OK or one of the codes above; kda_get_last_error() describes a
 * nonzero return.  No exception crosses this boundary.
 */
int kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
            float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
            const void* initial_state, int initial_state_dtype, void* final_state,
            int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
            int64_t T, int64_t H, int64_t K, int64_t V, void* workspace, size_t workspace_bytes,
            hipStream_t stream);

/*
 * kda_fwd_profiled -- kda_fwd that also records events[0..3] on `stream`:
 * before the scheduler, after it, after the chunk prep (on the fused path,
 * where prep and recurrence are one kernel, this is event [1] again) and
 * after the whole call, so a caller can time the stages with
 * hipEventElapsedTime.  Same arguments, checks and results as kda_fwd; the
 * four events are created and owned by the caller.  kda_fwd_ex gives
 * per-kernel events.
 */
int kda_fwd_profiled(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
                     const void* initial_state, int initial_state_dtype, void* final_state,
                     int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
                     int64_t T, int64_t H, int64_t K, int64_t V, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, hipEvent_t events[4]);

/*
 * kda_fwd_ex -- kda_fwd with the execution path, the chunk size and the
 * overlap of the two stages under the caller's control, and optional
 * per-kernel events.
 *
 * path: KDA_PATH_AUTO (the library's choice; with a 32- or 64-token chunk or
 * more than one part, the split path), KDA_PATH_SPLIT or KDA_PATH_FUSED (chunk 0 or
 * 16 and parts 0 or 1 only; otherwise KDA_EINVAL).  The workspace
 * must hold kda_fwd_workspace_bytes_ex(..., chunk, parts, path) bytes: the
 * split path keeps its chunk records there (about 864, 912 and 1032 B per
 * token-head at chunk 16, 32 and 64), the fused path only the per-sequence
 * tables.  (kda_fwd_workspace_bytes covers the 16- and 32-token forms only.)
 *
 * chunk: 0 (the library's choice, as kda_fwd), 16, 32 or 64 tokens per chunk.
 * The pages use 16 (P1 §二 2.1) so that the in-chunk decay factors stay in
 * range, against the 64 of Flash Linear Attention; the 32- and 64-token
 * kernels build each chunk from two or four 16-token blocks whose coupling
 * blocks need only bounded factors (the 64 x 64 inverse by block forward
 * substitution), and step the state a half or a quarter as often.  All
 * compute the same chunked form (any chunk size gives the exact recurrence up
 * to rounding); their results differ only in rounding.  Any other value
 * returns KDA_EINVAL.
 *
 * The token rows (B * T, flattened) are cut into `parts` consecutive ranges of
 * equal size.  The chunk-prep kernel of range p + 1 runs on `stream` while the
 * chunk recurrence of range p runs on a second stream that the library keeps
 * per device (created on first use, default priority); the recurrence hands
 * the state of every (sequence, head) from one range to the next through the
 * workspace in fp32, so the result equals the one-range result.  The call
 * still only enqueues work: `stream` waits for the second stream before
 * anything enqueued after the call.  parts = 0 lets the library choose
 * (kda_fwd does that; it chooses 1, since on MI355X the two kernels slow each
 * other down about as much as the overlap saves); values above 8 are clamped
 * to 8.  The split into two stages and their roles follow P1 §二
 * 2.2; overlapping them is this library's addition.
 *
 * events: NULL (num_events ignored) or kda_fwd_num_events(B, T, chunk, parts,
 * path) caller-owned events.  Split path (P = kda_fwd_parts(B, T, parts)):
 * 2 + 4 P events, [0] before the scheduler, [1] after it, [2 + 2p] / [3 + 2p]
 * before / after the prep kernel of part p (on `stream`), [2 + 2P + 2p] /
 * [3 + 2P + 2p] before / after the recurrence of part p (on the stream it runs
 * on).  Fused path: 4 events, [0] / [1] around the scheduler, [2] / [3] around
 * the fused kernel.  Library's choice (KDA_PATH_AUTO with 16-token chunks and
 * one part): 8 events, the split path's 6 and [6] / [7] around the fused
 * kernel.  A wrong count returns KDA_EINVAL.
 * Calls on one device that use the second stream are serialised on the host
 * by a per-device lock while they enqueue.
 */
int kda_fwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
               void* out, const float* A_log, const float* dt_bias, float lower_bound,
               const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
               const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
               int64_t V, void* workspace, size_t workspace_bytes, hipStream_t stream, int chunk,
               int parts, int path, hipEvent_t* events, int num_events);

/*
 * kda_fwd_precision -- a study entry point, not the hot path: kda_fwd on the
 * split path (16-token chunks, one part) with the chunk recurrence's or the
 * chunk prep's arithmetic changed to one of the alternatives P1 §二 2.1 and
 * 2.3 weigh, so their accuracy against an exact reference can be measured.
 *   KDA_PREC_DEFAULT: the library's arithmetic (state fp32 on chip, fp16
 *     MFMA operands with fp32 accumulation); equal to kda_fwd_ex(path = split).
 *   KDA_PREC_BF16_STATE: the state rounded to bf16 after every chunk update,
 *     as the pages store it between updates (the update itself stays fp32).
 *   KDA_PREC_BF16_INVERSE: E = T R with T (the record's inverse, rounded
 *     from fp16) and R in bf16, E rounded to bf16; the pages keep the inverse
 *     in fp16 for its precision.
 *   KDA_PREC_BF16_STATE_PRODUCTS: Khat Z and Qhat Z with the state copy and
 *     the record's -Khat and Qhat in bf16 instead of fp16.
 *   KDA_PREC_NEUMANN_FP16: the chunk prep forms the 16 x 16 inverse as the
 *     pages do (P1 §二 2.1, 2.3), the Neumann product (I - L)(I + L^2)(I + L^4)
 *     (I + L^8), exact since L is strictly lower, with every factor and
 *     product an fp16 matrix-core operand (fp32 accumulation), instead of
 *     forward substitution in fp32.
 * variant: any combination of these bits; anything else returns KDA_EINVAL.
 * Arguments, workspace (kda_fwd_workspace_bytes_ex(..., 16, 1,
 * KDA_PATH_SPLIT) bytes or more) and checks otherwise as kda_fwd.
 */
#define KDA_PREC_DEFAULT 0
#define KDA_PREC_BF16_STATE 1
#define KDA_PREC_BF16_INVERSE 2
#define KDA_PREC_BF16_STATE_PRODUCTS 4
#define KDA_PREC_NEUMANN_FP16 8
int kda_fwd_precision(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                      void* out, const float* A_log, const float* dt_bias, float lower_bound,
                      const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
                      const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
                      int64_t V, void* workspace, size_t workspace_bytes, hipStream_t stream, int variant);

/*
 * kda_fwd_fused_noalloc -- for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): kda_fwd_ex on the fused path (16-token
 * chunks, one part) with the workspace taken from a static device array of
 * the library, 320 KiB + 256 B per GPU, held until the process ends.  At most
 * 16384 sequences (num_seqs with cu_seqlens, else B); more returns
 * KDA_EINVAL before any HIP call.  Arguments, checks and results otherwise as
 * kda_fwd_ex(path = KDA_PATH_FUSED): bit for bit the same outputs.  The call
 * allocates nothing and frees nothing; the first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress).
 * All calls on one GPU share its array, which keeps the last call's tables:
 * calls that overlap on one GPU (other streams, other threads) race and give
 * undefined results; serialise them.  A rejected cu_seqlens leaves out and
 * final_state untouched; its status word is not readable by the caller.
 */
int kda_fwd_fused_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                          void* out, const float* A_log, const float* dt_bias, float lower_bound,
                          const void* initial_state, int initial_state_dtype, void* final_state,
                          int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                          int64_t H, int64_t K, int64_t V, hipStream_t stream);

/* Number of parts kda_fwd_ex uses for these sizes and `parts` request (0 on bad input). */
int kda_fwd_parts(int64_t B, int64_t T, int parts);

/* Path that kda_fwd_ex takes for these requests: KDA_PATH_SPLIT,
   KDA_PATH_FUSED, KDA_PATH_AUTO (chosen on the device, see
   kda_fwd_path_taken), or -1 if they are invalid together. */
int kda_fwd_path(int chunk, int parts, int path);

/* Path (KDA_PATH_SPLIT or KDA_PATH_FUSED) that the last call using
   `workspace` ran.  Synchronises `stream` first; for tests and tools. */
int kda_fwd_path_taken(const void* workspace, hipStream_t stream, int* path);

/* Events kda_fwd_ex takes for these sizes and requests (0 on bad input). */
int kda_fwd_num_events(int64_t B, int64_t T, int chunk, int parts, int path);

/*
 * kda_fwd_segmented -- kda_fwd with every sequence cut into `segments` pieces
 * whose chunk chains run side by side, for calls with few long sequences and
 * few heads, where one (sequence, head) chain per value tile cannot fill the
 * chip.  P1 §二 2.2 keeps the recurrence stage parallel over heads only and
 * shows the long unfragmented sequence as the slow case; cutting a sequence
 * is this library's addition, not on the pages.
 *
 * Over a segment the update of P1 §一 maps the starting state affinely,
 * S_end = A S_start + B, with A the product of (I - beta_t kn_t kn_t^T)
 * diag(exp(a_t)) over the segment's tokens and B its end state from a zero
 * start.  The call builds the chunk records of all segments of all sequences
 * once (the split path's scheduler and prep kernels) and runs the chunk
 * recurrence three times over them: with the values from a zero start
 * (giving B) and with zero values from the identity (giving A), both in one
 * launch that writes no outputs, and, after a small kernel has composed per
 * (sequence, head) S_start(0) = initial state,
 * S_start(j + 1) = A_j S_start(j) + B_j (the last composition is the final
 * state), with the values from each segment's true start.  Segments are
 * ceil(len / segments) tokens rounded up to whole 16-token chunks, the last
 * ones shorter or empty; an empty segment passes its state through exactly.
 * The result equals kda_fwd's up to rounding: the states between segments are
 * kept in fp32, and each composition rounds its operands to fp16 as the
 * recurrence does every chunk.
 *
 * Arguments, checks, states (the same buffer allowed for both) and the device
 * status word are those of kda_fwd.  segments: 1 .. 4096, or 0 for the
 * library's choice (kda_fwd_segments); 1 is exactly kda_fwd.  workspace:
 * 256-byte aligned, of at least kda_fwd_segmented_workspace_bytes(...) bytes
 * with the same `segments` (kda_fwd's workspace for the segments, then per
 * (segment, head) the 128 x 128 transition A in fp16 and two fp32 128 x 128
 * states); kda_fwd_check_status reads it as it reads kda_fwd's.
 * A's entries lie in [-1, 1] (each factor is a contraction), so it is kept in
 * fp16, and the composition uses fp16 operands with fp32 accumulation.
 */
int kda_fwd_segmented(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                      void* out, const float* A_log, const float* dt_bias, float lower_bound,
                      const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
                      const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K,
                      int64_t V, int segments, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The segment count kda_fwd_segmented takes for segments = 0: the largest
   power of two that keeps at most 128 (segment, head) chains and segments of
   at least 512 tokens (the mean length with cu_seqlens), or 1 (no cut) when
   that is below 4.  0 on bad sizes. */
int kda_fwd_segments(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens);

/* Workspace bytes kda_fwd_segmented needs (0 on bad sizes). */
size_t kda_fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens,
                                         int segments);

/*
 * kda_decode -- enqueue one recurrent step (one new token per sequence) on
 * `stream`: the token-by-token recurrence of P1 §一 with the activations of
 * kda_fwd, no chunking and no workspace.
 *
 * q, k, g, v: bf16 [N][H][128] (token n of sequence n, i.e. kda_fwd's
 * [B, T, H, 128] with B = N, T = 1); beta: bf16 [N][H]; out: bf16 [N][H][128];
 * A_log, dt_bias, lower_bound, scale and the states ([N][H][V][K], bf16 or
 * fp32, NULL = zero state / not written, the same buffer allowed for both) as
 * for kda_fwd.  Each (sequence, head) state is read and written once, so the
 * call is bound by the state bytes.  Argument errors are caught on the host
 * before any HIP call, with the codes of kda_fwd.
 */
int kda_decode(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
               void* out, const float* A_log, const float* dt_bias, float lower_bound,
               const void* initial_state, int initial_state_dtype, void* final_state, int final_state_dtype,
               int64_t N, int64_t H, int64_t K, int64_t V, hipStream_t stream);

/*
 * Workspace bytes that suit kda_fwd (the segmented form it may take
 * included) and every kda_fwd_ex path and chunk size for these sizes (0 if
 * the sizes are invalid).  num_seqs is ignored when
 * has_cu_seqlens is 0 (then N = B).
 */
size_t kda_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t num_seqs,
                               int has_cu_seqlens);

/* Workspace bytes for one kda_fwd_ex configuration (chunk, parts, path as
   there; 0 if invalid).  The fused path needs only the per-sequence tables. */
size_t kda_fwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens,
                                  int chunk, int parts, int path);

/* Thread-local description of the last nonzero return on this thread. */
const char* kda_get_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

/*
 * kda_fwd_check_status -- read the device status word that the last kda_fwd
 * using `workspace` wrote (KDA_STATUS_*).  Synchronises `stream` first; meant
 * for tests and debugging, not for the hot loop.
 */
int kda_fwd_check_status(const void* workspace, hipStream_t stream, int* status);

/*
 * Workspace layout for chunk = 16, 32 or 64, for tests that decode the chunk records:
 * offsets[0] = chunk table (int32 triples {sequence, first token row, length}),
 * offsets[1] = per-sequence table (int32 quadruples {first chunk, chunk count,
 *              first token row, length}),
 * offsets[2] = work order (int32 [N], sequences longest first),
 * offsets[3] = chunk records, chunk-major: record (chunk c, head h) at
 *              offsets[3] + (c * H + h) * offsets[4],
 * offsets[4] = bytes per record, offsets[5] = chunk capacity (floor(B*T/chunk) + N),
 * offsets[6] = total bytes.  Returns KDA_OK or KDA_EINVAL.
 * Record layout for chunk 16 (bytes): [0, 4096) Qhat fp16 [16][128]; [4096, 8192) -Khat fp16
 * [16][128]; both with the channels of each 32-block stored in the order
 * {0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31}; [8192, 12288) Kbar fp16
 * [16][128] (token-major, natural channel order); [12288, 12800) T^T fp16
 * [16][16]; [12800, 13312) Mqk^T fp16 [16][16]; [13312, 13824) gamma fp32 [128],
 * channel c = 64 r + 16 a + 4 b + i stored at slot 2 (16 b + 4 a + i) + r.
 * Record layout for chunk 32 (bytes): [0, 8192) Qhat fp16 [32][128] and
 * [8192, 16384) -W fp16 [32][128], channels as above; [16384, 24576) Kbar fp16
 * [32][128] (token-major, natural order); [24576, 26624) T fp16 [32][32] and
 * [26624, 28672) Mqk fp16 [32][32], both row-major with the columns of each row
 * in the order {0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31};
 * [28672, 29184) gamma fp32 [128] as above.
 * Record layout for chunk 64 (bytes): [0, 16384) Qhat fp16 [64][128] and
 * [16384, 32768) -W fp16 [64][128], channels as above; [32768, 49152) Kbar fp16
 * [64][128] (token-major, natural order); [49152, 57344) T and [57344, 65536)
 * Mqk, fp16, each as eight blocks of 16 rows x 32 columns, block (t, u) (rows
 * 16t .. 16t + 15, token columns 32u .. 32u + 31 in the order above) at
 * (2t + u) * 1024 bytes, the blocks above the diagonal zero; [65536, 66048)
 * gamma fp32 [128] as above.
 */
int kda_workspace_layout(int64_t B, int64_t T, int64_t H, int64_t num_seqs, int has_cu_seqlens, int chunk,
                         int64_t offsets[7]);

/*
 * kda_debug_prep -- test-only: enqueue the scheduler and the split path's chunk-prep kernels
 * alone (same arguments as kda_fwd minus v, out and the states, plus the
 * chunk size, 16, 32 or 64), leaving the chunk table and records in `workspace`
 * for inspection.
 */
int kda_debug_prep(const void* q, const void* k, const void* g, const void* beta, float scale,
                   const float* A_log, const float* dt_bias, float lower_bound,
                   const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H,
                   int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream, int chunk);

/*
 * kda_debug_set_spin_limit -- test-only: waits between the waves of a
 * workgroup (the split path's recurrence at 64 or 128 value columns per
 * workgroup, and the fused kernel) give up after `polls` polls in the launches
 * that follow, and report KDA_STATUS_SYNC_TIMEOUT; 0 makes every such wait give up at once (the
 * kernels still finish, with meaningless outputs).  A negative value restores
 * the default (2^21 polls).  Process-wide, applies to every device; not meant
 * to be called while another thread launches.  Returns KDA_OK.
 */
int kda_debug_set_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* KDA_MI355X_H */
