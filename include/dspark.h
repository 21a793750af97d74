/*
 * libdspark: the per-step draft -> schedule -> verify hot path of DSpark
 * speculative decoding, for AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * Sources of the operations (web pages; cited by title and section):
 *   [EXP]  "DSpark: speculative decoding that fixes suffix quality and
 *          production verification waste" (papers.franksyz.com explainer),
 *          sections 2-5 and 7-13.
 *   [PR]   llama.cpp PR #25173 "spec: add DSpark speculative decoding",
 *          description and review thread.
 *
 * One step for R requests, block size gamma, vocabulary V, Markov rank r:
 *   dspark_draft_block  drafts gamma tokens per request left to right;
 *   dspark_schedule     computes survival and picks the verify rows;
 *   (the caller runs the target model over those rows)
 *   dspark_verify       accepts / rejects and emits one correction or bonus.
 *
 * Conventions shared by every call:
 *   - Every array pointer is a DEVICE pointer (memory of the current HIP
 *     device), except the argument struct itself, which lives on the host.
 *   - All arrays are dense, row-major, with the shapes given below.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates or frees memory and keeps no pointer after returning.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  No call synchronises the host or
 *     copies device data to the host.  Every output size is known on the host
 *     before the call.
 *   - Errors: argument checks (NULL pointers, sizes, limits, alignment,
 *     struct_size, workspace size) run on the host before anything is
 *     enqueued; on failure a nonzero dspark_status is returned and nothing is
 *     enqueued.  A failed kernel launch returns DSPARK_ERR_HIP.  Device data
 *     (token ids, logits, offsets, probabilities) is not inspected on the
 *     host; out-of-range ids and offsets are clamped inside the kernels so no
 *     access leaves its buffer, but the results are then unspecified.
 *   - Device input checks (debug): with DSPARK_CHECK_INPUTS in `flags`, a
 *     call first runs a small kernel that inspects its device inputs (token
 *     ids, uniforms, confidences, verify row offsets) and writes what it
 *     found as DSPARK_BAD_* bits into the error word at the start of the
 *     call's workspace; the call's other kernels run as usual.
 *     dspark_check() synchronises the stream and reads that word back.  A
 *     block size or verify length that does not match the call is thereby
 *     reported instead of silently changing the results ([PR] automated
 *     review: a non-uniform block must not be inferred silently, a degraded
 *     result must not be silent, a missing input must be an error).
 *   - No C++ exception crosses this interface and nothing is printed.
 *   - Calls that share a workspace must not overlap in time.
 *   - Argument structs are versioned: set struct_size = sizeof(the struct).
 */
#ifndef DSPARK_H_
#define DSPARK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 3

/* limits checked on the host */
#define DSPARK_MAX_GAMMA 16          /* block size gamma in [1, 16]                 */
#define DSPARK_MAX_RANK 512          /* Markov rank r in [8, 512], r % 8 == 0       */
#define DSPARK_MAX_VOCAB (1 << 30)   /* V in [1, 2^30]                              */
#define DSPARK_SCHED_KEYS_PER_THREAD 16  /* dspark_schedule: ceil(R/1024)*gamma <= 16 */
#define DSPARK_CAPACITY_MAX_CANDIDATES 16384  /* dspark_capacity: R * gamma <= 16384 */

typedef enum dspark_status {
  DSPARK_OK = 0,
  DSPARK_ERR_NULL = 1,        /* a required pointer is NULL                        */
  DSPARK_ERR_SHAPE = 2,       /* a size is out of range                            */
  DSPARK_ERR_DTYPE = 3,       /* unknown weight dtype                              */
  DSPARK_ERR_ALIGN = 4,       /* a pointer is not aligned as required              */
  DSPARK_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  DSPARK_ERR_UNSUPPORTED = 6, /* valid but outside this library's limits           */
  DSPARK_ERR_ABI = 7,         /* struct_size does not match this library          */
  DSPARK_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed        */
  DSPARK_ERR_INPUT = 9        /* dspark_check: a device input check failed         */
} dspark_status;

/* Bits of the `flags` field of the argument structs. */
#define DSPARK_CHECK_INPUTS 1u       /* run the device input checks (debug)          */

/* Bits of the error word that dspark_check() returns (the start of the
 * workspace of a call made with DSPARK_CHECK_INPUTS). */
#define DSPARK_BAD_TOKEN (1u << 0)      /* an anchor or drafted token outside [0, V)  */
#define DSPARK_BAD_UNIFORM (1u << 1)    /* a uniform outside [0, 1), or NaN          */
#define DSPARK_BAD_LENGTH (1u << 2)     /* verify rows: a request owns fewer than 1 or
                                           more than gamma + 1 rows (l outside
                                           [0, gamma]), or the offsets leave
                                           [0, n_rows]                               */
#define DSPARK_BAD_CONFIDENCE (1u << 3) /* a confidence outside [0, 1], or NaN       */
/* Size of the header that holds the error word at the start of every
 * workspace (the rest of the workspace follows it). */
#define DSPARK_WORKSPACE_HEADER 256

/* Element type of the Markov factors W1, W2. */
typedef enum dspark_wdtype {
  DSPARK_W_F32 = 0,           /* IEEE binary32                                     */
  DSPARK_W_BF16 = 1           /* bfloat16 bit patterns (uint16)                    */
} dspark_wdtype;

/* The drafter's sequential head ([EXP] section 7 names a Markov head and an
 * RNN head that carries a longer in-block state; the pages give the RNN
 * head no equations, and this library takes the Elman recurrence below). */
typedef enum dspark_head {
  DSPARK_HEAD_MARKOV = 0,     /* h_k = W1[prev_k]                                  */
  DSPARK_HEAD_RNN = 1         /* h_k = act(A h_{k-1} + W1[prev_k]), h_{-1} = 0     */
} dspark_head;

/* Activation of the RNN head. */
typedef enum dspark_act {
  DSPARK_ACT_IDENTITY = 0,
  DSPARK_ACT_TANH = 1
} dspark_act;

/* --------------------------------------------------------------------------
 * dspark_draft_block: draft one block of gamma tokens per request.
 *
 * [EXP] section 7: drafter logits are base logits U_k plus a prefix-dependent
 * bias B_k; the Markov head's bias depends only on the previous sampled token
 * and is a low-rank factorisation instead of a V x V transition table.
 * [PR] description: the block is anchor-first (position 0 already predicts
 * the first draft token) and sampled left to right with
 * bias(prev) = markov_w2 . markov_w1[prev], computed on the device.
 * [EXP] section 6: a parallel backbone produces U for all positions; the
 * light sequential head corrects each next position.
 *
 * For k = 0 .. gamma-1, sequentially (y[:, k-1] feeds position k):
 *   prev[r]  = anchor[r] if k == 0 else y[r, k-1]
 *   h[r, k]  = W1[prev[r]]                            (DSPARK_HEAD_MARKOV)
 *              act(A h[r, k-1] + W1[prev[r]]), h[r, -1] = 0  (DSPARK_HEAD_RNN)
 *   s[r, v]  = U[r, k, v] + sum_j W2[v, j] * h[r, k, j]
 *   greedy (temp[r] <= 0 or NaN):
 *     y[r, k] = lowest index v with maximal s[r, v]; q_tok = 1;
 *     q_stats = (max_v s, 1)
 *   sampled (temp[r] = T > 0; T is used clamped to [1e-30, 1e30], so
 *   T = +inf samples uniformly over the entries that are not -inf):
 *     x = s / T, m = max x, Z = sum_v exp(x_v - m);
 *     y[r, k] = first v (in index order) whose inclusive cumulative sum of
 *               exp(x - m) exceeds u_draft[r, k] * Z (never a zero-mass entry);
 *     q_tok[r, k] = exp(x_y - m) / Z;  q_stats[r, k] = (max_v s, Z)
 *
 * Arguments (device arrays unless stated):
 *   R, gamma, V, rank   host ints; R >= 0 (R == 0 is a no-op), gamma in
 *                       [1, DSPARK_MAX_GAMMA], V in [1, DSPARK_MAX_VOCAB],
 *                       rank in [8, DSPARK_MAX_RANK] with rank % 8 == 0.
 *   wdtype              dspark_wdtype of W1 and W2.
 *   flags               0, or DSPARK_CHECK_INPUTS (checks anchor and u_draft).
 *   U        float [R, gamma, V]  base logits; 16-byte aligned.  Each entry
 *                                 is finite or -inf (a masked token), and
 *                                 every row of U + B has a finite entry;
 *                                 +inf and NaN logits are outside this
 *                                 contract (results are then undefined).
 *   W1, W2   wdtype [V, rank]     Markov factors (markov_w1, markov_w2);
 *                                 16-byte aligned; finite.
 *   anchor   int32 [R]            last committed token (prev for k = 0), in
 *                                 [0, V); the kernels clamp a token index
 *                                 into that range before any use.
 *   temp     float [R]            per-request temperature; <= 0 => greedy.
 *   u_draft  float [R, gamma]     uniforms in [0, 1) (read by sampled rows).
 *   y        int32 [R, gamma]     out: drafted tokens.
 *   q_tok    float [R, gamma]     out: drafter probability of y.
 *   q_stats  float [R, gamma, 2]  out: (max_v s, Z) per position, consumed by
 *                                 dspark_verify to rebuild q on a rejection.
 *   workspace, workspace_bytes    scratch of at least
 *                                 dspark_draft_workspace_size() bytes,
 *                                 256-byte aligned (the segment records; with
 *                                 the RNN head on the 16-row path also a
 *                                 fragment-packed copy of A, made by the
 *                                 call when W2_packed is given).
 *   stream   hipStream_t as void*.
 *   prof_events  optional (NULL normally): host array of 2*gamma hipEvent_t
 *                handles (created with timing enabled); events 2k / 2k+1 are
 *                attached to the dispatch of the fused bias + softmax kernel
 *                of position k (hipExtLaunchKernel start / stop events), so
 *                their interval is that kernel's execution time alone.
 *   W2_packed    optional (NULL normally): the output of dspark_pack_w2 for
 *                this W2, 16-byte aligned; read instead of W2 by the fused
 *                kernel when the batch takes the 16-row path (bf16, R <= 64).
 *   W2_packed_bytes  size of the W2_packed buffer; at least
 *                dspark_w2_packed_bytes(V, rank) when W2_packed is given
 *                (DSPARK_ERR_WORKSPACE otherwise).
 *   head     dspark_head.  DSPARK_HEAD_RNN needs bf16 weights and R <= 64
 *            (the 16-row path; DSPARK_ERR_UNSUPPORTED otherwise); an unknown
 *            head or act is DSPARK_ERR_UNSUPPORTED.
 *   act      dspark_act of the RNN head (ignored by the Markov head).
 *   A        RNN head: wdtype [rank, rank] recurrence matrix, row j gives
 *            output j (z_j = sum_i A[j, i] h_i); 16-byte aligned.  Else NULL.
 *   h        RNN head: float [R, gamma, rank] out, 16-byte aligned: the
 *            states h[r, k], which dspark_verify reads back.  They are
 *            computed in fp32 and stored as double-bf16 values (the sum of
 *            two bf16 numbers, 16 significant bits), the form in which the
 *            fused bias kernel feeds them to the bf16 matrix cores exactly.
 *            Else NULL.
 * -------------------------------------------------------------------------- */
typedef struct dspark_draft_args {
  uint32_t struct_size;
  int32_t R, gamma, V, rank;
  int32_t wdtype;
  uint32_t flags;
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* anchor;
  const float* temp;
  const float* u_draft;
  int32_t* y;
  float* q_tok;
  float* q_stats;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  void* const* prof_events;
  const void* W2_packed;
  size_t W2_packed_bytes;
  int32_t head;
  int32_t act;
  const void* A;
  float* h;
} dspark_draft_args;

/* --------------------------------------------------------------------------
 * dspark_schedule: survival and the causal, prefix-closed verify schedule.
 *
 * [EXP] section 8: the confidence head estimates the conditional acceptance
 * c[r, k]; the scheduler uses the cumulative survival a[r, k] (probability
 * the prefix survives).  Section 5: a suffix position's value is a product
 * of conditional acceptance rates.  Section 9: the chosen work is
 * prefix-closed (no verifying position 5 alone).  Section 10: capacity K is
 * fixed ahead of time; the current cumulative confidence picks a top-K
 * prefix selection inside it.  Section 4: admission must not read the
 * drafted tokens (this call's decision reads only c and K).  Section 13: the
 * variable-length verify tokens are flattened into contiguous rows with
 * per-sequence markers instead of padding.
 *
 *   a[r, 0] = c'[r, 0], a[r, k] = fl32(a[r, k-1] * c'[r, k]) with
 *             c' = c clamped to [0, 1] (NaN -> 0) and -0 written as +0;
 *   Kc      = min(max(K, 0), R * gamma);
 *   the Kc candidates (r, k) first in the order (a descending, k ascending,
 *   r ascending) are selected; l[r] = number selected for request r (always a
 *   prefix 0 .. l[r]-1 because a is non-increasing in k);
 *   row_offsets[0] = 0, row_offsets[r+1] = row_offsets[r] + l[r] + 1;
 *   for row i = row_offsets[r] + j, j = 0 .. l[r]:
 *     row_req[i] = r, row_pos[i] = j,
 *     row_tok[i] = anchor[r] if j == 0 else y[r, j-1]   (the token fed to the
 *     target at that row; row j verifies draft j, row l[r] is the bonus row);
 *   expected_tokens = R + sum of a over the selected candidates.
 *
 * Arguments (device arrays unless stated):
 *   R, gamma   host ints; R >= 0, gamma in [1, DSPARK_MAX_GAMMA],
 *              ceil(R / 1024) * gamma <= DSPARK_SCHED_KEYS_PER_THREAD.
 *   K          host int64 capacity in draft positions (any value; clamped).
 *   flags      0, or DSPARK_CHECK_INPUTS (checks that c is in [0, 1] and that
 *              anchor and y are not negative; this call knows no V).
 *   c          float [R, gamma]  per-position acceptance estimates.
 *   anchor     int32 [R]; y int32 [R, gamma] (drafted tokens; only copied
 *              into row_tok, never read by the decision).
 *   a          float [R, gamma]  out: survival.
 *   l          int32 [R]         out: verified draft count per request.
 *   row_offsets int32 [R + 1]    out.
 *   row_req, row_pos, row_tok  int32 [dspark_schedule_rows(R, gamma, K)] out.
 *   expected_tokens  float [1]   optional out (may be NULL).
 *   workspace, workspace_bytes  dspark_schedule_workspace_size() bytes,
 *              256-byte aligned: none (NULL, 0) without DSPARK_CHECK_INPUTS,
 *              the error-word header with it.
 *   stream     hipStream_t as void*.
 * -------------------------------------------------------------------------- */
typedef struct dspark_schedule_args {
  uint32_t struct_size;
  int32_t R, gamma;
  int64_t K;
  uint32_t flags;
  const float* c;
  const int32_t* anchor;
  const int32_t* y;
  float* a;
  int32_t* l;
  int32_t* row_offsets;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t* row_tok;
  float* expected_tokens;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
} dspark_schedule_args;

/* --------------------------------------------------------------------------
 * dspark_verify: accept / reject drafted tokens against target logits.
 *
 * [EXP] section 2: the target verifies the prefix under a causal mask;
 * verification runs left to right and after the first rejection the later
 * drafts are discarded; if all are accepted a bonus token comes from the
 * target's next distribution, otherwise a correction from the residual.
 * Section 3: accept v with probability min(1, p(v)/q(v)); the correction
 * takes only the target's mass in excess of the drafter, max(0, p - q)
 * normalised (resampling from full p would double-count the overlap).
 * [PR] "Losslessness": greedy decoding stays identical to target-only
 * greedy.
 *
 * Request r owns target rows row_offsets[r] .. row_offsets[r+1]-1, so its
 * verify length is l = rows - 1 (0 <= l <= gamma); row j holds the target
 * logits t_j for draft position j, row l is the bonus position.
 *   greedy (temp[r] <= 0 or NaN):
 *     accept y_j iff y_j is the lowest-index argmax of t_j; p_tok = 1 or 0;
 *     n = first rejected j (else l); out_tok = lowest-index argmax of t_n.
 *   sampled (T = temp[r] > 0, clamped as in dspark_draft_block):
 *     p_j = softmax(t_j / T); p_tok[r, j] = p_j(y_j);
 *     accept iff u_accept[r, j] < p_tok[r, j] / q_tok[r, j];
 *     n = first rejected j, else l;
 *     n < l: q_n = softmax((U[r, n] + W2 . h[r, n]) / T) rebuilt with the
 *            draft's h (Markov head: W1[prev], prev = anchor (n = 0) or
 *            y[r, n-1]; RNN head: the state array) and q_stats[r, n];
 *            out_tok = inverse-CDF draw with u_final[r] from max(0, p_n - q_n)
 *            (from p_n if that has no mass);
 *     n = l: out_tok = inverse-CDF draw with u_final[r] from p_l (bonus).
 *   Emitted tokens for the step: y[r, 0 .. n-1] followed by out_tok[r].
 *   p_tok[r, j] = 0 for j >= l.
 *
 * Arguments (device arrays unless stated):
 *   R, gamma, V, rank, wdtype  as for dspark_draft_block.
 *   flags      0, or DSPARK_CHECK_INPUTS (checks row_offsets, anchor, y,
 *              u_accept and u_final).
 *   n_rows     host int64: total rows = row_offsets[R]; R <= n_rows <=
 *              R * (gamma + 1).
 *   target     float [n_rows, V]  target logits; 16-byte aligned; finite or
 *                                 -inf, with a finite entry in every row
 *                                 (as for U).
 *   row_offsets int32 [R + 1]     (from dspark_schedule, or r*(gamma+1) for
 *                                  fixed-length verify).
 *   U, W1, W2, anchor, temp       the inputs given to dspark_draft_block.
 *   y, q_tok, q_stats             outputs of dspark_draft_block.
 *   u_accept   float [R, gamma]   uniforms in [0, 1).
 *   u_final    float [R]          uniform in [0, 1).
 *   n_accept   int32 [R]          out: accepted draft count n.
 *   out_tok    int32 [R]          out: correction or bonus token.
 *   p_tok      float [R, gamma]   out: target probability of each draft.
 *   workspace, workspace_bytes    >= dspark_verify_workspace_size(); 256-byte
 *                                 aligned.
 *   stream     hipStream_t as void*.
 *   W2_packed, W2_packed_bytes  optional, as for dspark_draft_block (read by
 *              the residual pass of the 16-row path).
 *   head       the head the block was drafted with (same limits).
 *   h          RNN head: the float [R, gamma, rank] states written by
 *              dspark_draft_block, 16-byte aligned.  Else NULL.
 * -------------------------------------------------------------------------- */
typedef struct dspark_verify_args {
  uint32_t struct_size;
  int32_t R, gamma, V, rank;
  int32_t wdtype;
  uint32_t flags;
  int64_t n_rows;
  const float* target;
  const int32_t* row_offsets;
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* anchor;
  const float* temp;
  const int32_t* y;
  const float* q_tok;
  const float* q_stats;
  const float* u_accept;
  const float* u_final;
  int32_t* n_accept;
  int32_t* out_tok;
  float* p_tok;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  const void* W2_packed;
  size_t W2_packed_bytes;
  int32_t head;
  const float* h;
} dspark_verify_args;

/* Workspace bytes needed by a call with these arguments (only the size
 * fields and flags are read).  Returns DSPARK_OK and writes *bytes, or an
 * error status for invalid sizes.  Draft and verify workspaces start with
 * the DSPARK_WORKSPACE_HEADER bytes of the error word; the schedule calls
 * need a workspace (that header alone) only with DSPARK_CHECK_INPUTS, and
 * report 0 bytes otherwise. */
int dspark_draft_workspace_size(const dspark_draft_args* args, size_t* bytes);
int dspark_verify_workspace_size(const dspark_verify_args* args, size_t* bytes);
int dspark_schedule_workspace_size(const dspark_schedule_args* args, size_t* bytes);

/* --------------------------------------------------------------------------
 * dspark_check: result of the device input checks of the last call that
 * used `workspace` with DSPARK_CHECK_INPUTS (debug only: it synchronises).
 *
 * Waits for `stream` (hipStream_t as void*), then copies the error word at
 * the start of the workspace to the host.  Returns DSPARK_OK when it is 0,
 * DSPARK_ERR_INPUT when some DSPARK_BAD_* bit is set, DSPARK_ERR_NULL for a
 * NULL workspace, DSPARK_ERR_HIP if the wait or the copy fails.  *bits (may
 * be NULL) receives the word.  Every call that uses a draft or verify
 * workspace rewrites the word (0 when it was made without the flag), so a
 * check reports the call that ran last on that workspace.
 * -------------------------------------------------------------------------- */
int dspark_check(const void* workspace, void* stream, uint32_t* bits);

/* --------------------------------------------------------------------------
 * dspark_schedule_cutoff: survival and the static confidence-cutoff schedule.
 *
 * [PLAN] "Approach", step 5: confidence scheduling first evaluates a static
 * confidence cutoff, before any load-aware scheduler.  [LCPP] "Confidence
 * Evaluation": the conf_min setting (measured at 0.0, 0.3 and 0.6).  Each
 * request verifies its leading drafted positions while each position's own
 * confidence reaches conf_min, and stops at the first that does not: a
 * per-request rule, prefix-closed by construction, with no global capacity.
 * Like dspark_schedule, the decision reads only c, never the drafted tokens
 * ([EXP] section 4).
 *
 *   c'[r, k]  = c clamped to [0, 1] (NaN -> 0), as for survival;
 *   l[r]      = the largest m in 0..gamma with c'[r, k] >= conf_min for
 *               every k < m (fp32 comparison);
 *   a, row_offsets, row_req, row_pos, row_tok and expected_tokens are then
 *   defined exactly as by dspark_schedule for this l.
 *
 * conf_min <= 0 verifies every position (the fixed-length schedule);
 * conf_min > 1 verifies none (target-only decoding).
 *
 * Arguments: as dspark_schedule_args (flags and workspace included),
 * without K and with
 *   conf_min   host float, not NaN (DSPARK_ERR_SHAPE otherwise).
 *   row_req, row_pos, row_tok  int32 [R * (gamma + 1)] out: room for the
 *              largest schedule (R + sum l[r] rows are written; the number is
 *              row_offsets[R]).
 * -------------------------------------------------------------------------- */
typedef struct dspark_cutoff_args {
  uint32_t struct_size;
  int32_t R, gamma;
  float conf_min;
  uint32_t flags;
  const float* c;
  const int32_t* anchor;
  const int32_t* y;
  float* a;
  int32_t* l;
  int32_t* row_offsets;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t* row_tok;
  float* expected_tokens;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
} dspark_cutoff_args;

/* Workspace bytes of dspark_schedule_cutoff: 0, or the error-word header with
 * DSPARK_CHECK_INPUTS (as dspark_schedule_workspace_size). */
int dspark_cutoff_workspace_size(const dspark_cutoff_args* args, size_t* bytes);


/* --------------------------------------------------------------------------
 * dspark_capacity: hardware-aware capacity K for a later step.
 *
 * [EXP] section 9: the scheduler should pick the prefix-closed verify work
 * that maximises the expected effective output times the engine's measured
 * step rate SPS(B) for a batch of B query tokens (step-shaped over the
 * graph-capture sizes); candidates are added in order of cumulative
 * survival and the greedy stops when that product no longer improves.
 * Section 10: so that the physical batch shape is known ahead and no host
 * round trip stalls the step, the capacity for an upcoming step is predicted
 * from the confidence of an earlier step (lagged); a_lag is that earlier
 * step's survival (the a output of dspark_schedule), and the K written here
 * is meant to be read back asynchronously and passed to dspark_schedule of a
 * later step.
 *
 *   v_1 >= v_2 >= ...  the R * gamma values of a_lag clamped to [0, 1]
 *                      (NaN -> 0), sorted descending;
 *   E(K)     = R + fl64(v_1 + ... + v_K)    (the exact sum rounded once to
 *              fp64, then an fp64 add; the expected tokens of the schedule
 *              with capacity K: R bonus/correction tokens plus survival);
 *   Theta(K) = E(K) * SPS[R + K]            (fp64 multiply; the batch has R
 *              anchor rows and K draft rows);
 *   kmax     = min(R * gamma, n_sps - 1 - R);
 *   K        = the first K in 0 .. kmax-1 with NOT Theta(K+1) > Theta(K),
 *              else kmax (greedy: add while Theta strictly improves).
 * The result depends only on the multiset of values, not on their order.
 *
 * Arguments (device arrays unless stated):
 *   R, gamma   host ints; R >= 0, gamma in [1, DSPARK_MAX_GAMMA],
 *              R * gamma <= DSPARK_CAPACITY_MAX_CANDIDATES.
 *   n_sps      host int: entries of sps; n_sps >= R + 1 (DSPARK_ERR_SHAPE
 *              otherwise: the table must at least cover the anchor rows).
 *   a_lag      float [R, gamma]  survival of an earlier step (may be NULL
 *              when R == 0).
 *   sps        float [n_sps]     steps per second of a verify batch of B
 *              rows, B = 0 .. n_sps-1 (any positive unit; scaling the table
 *              by a power of two never changes K).
 *   K          int32 [1]   out.
 *   expected   double [1]  optional out: E(K).
 *   theta      double [1]  optional out: Theta(K).
 *   stream     hipStream_t as void*.
 * One workgroup; no workspace.
 * -------------------------------------------------------------------------- */
typedef struct dspark_capacity_args {
  uint32_t struct_size;
  int32_t R, gamma;
  int32_t n_sps;
  const float* a_lag;
  const float* sps;
  int32_t* K;
  double* expected;
  double* theta;
  void* stream;
} dspark_capacity_args;

int dspark_capacity(const dspark_capacity_args* args);

/* --------------------------------------------------------------------------
 * Sequential temperature scaling of the confidence head ("STS").
 *
 * [EXP] section 8: the scheduler multiplies survival by the hardware
 * throughput curve, so a confidence head that ranks well but is
 * over-confident in absolute value makes wrong capacity decisions; the
 * cumulative probabilities are therefore corrected by a posterior
 * temperature calibration, position by position from left to right.
 *
 * dspark_sts_fit: one temperature per block position from calibration data.
 *   Calibration block i (of N) has confidence logits z[i, 0..gamma-1] and
 *   n_acc[i] accepted drafts (clamped to [0, gamma]).  It reached position k
 *   iff n_acc[i] >= k (every earlier draft accepted) and was accepted there
 *   iff n_acc[i] > k.  For each k, over the blocks that reached k:
 *     beta_k = the root of g(beta) = sum z_ik (sigmoid(beta z_ik) - y_ik)
 *              (the maximum-likelihood inverse temperature of
 *              P(accept k | reached k) = sigmoid(beta z); g is
 *              non-decreasing in beta), in [2^-8, 2^8]: 2^-8 if
 *              g(2^-8) >= 0, 2^8 if g(2^8) <= 0 (no sign change);
 *     beta_k = 1 when no block reached k or all its logits are 0;
 *     tau[k] = fp32(1 / beta_k).
 *   Logits are clamped to [-64, 64], NaN -> 0.  Each position's fit uses
 *   only the blocks that reached it, so the product of the calibrated
 *   conditional rates estimates the survival P(n_acc > k).
 *   Arguments: N >= 0 host int; gamma in [1, DSPARK_MAX_GAMMA];
 *   z float [N, gamma]; n_acc int32 [N]; tau float [gamma] out.
 *   One workgroup per position; calibration is an offline step.
 *
 * dspark_sts_apply: calibrated confidence for a batch,
 *   c[r, k] = fp32(sigmoid(z[r, k] / tau[k])) evaluated in fp64 (logits
 *   clamped as above), the c input of dspark_schedule.
 *   Arguments: R >= 0 host int; gamma in [1, DSPARK_MAX_GAMMA];
 *   z float [R, gamma]; tau float [gamma] (> 0); c float [R, gamma] out.
 * -------------------------------------------------------------------------- */
typedef struct dspark_sts_fit_args {
  uint32_t struct_size;
  int32_t N, gamma;
  const float* z;
  const int32_t* n_acc;
  float* tau;
  void* stream;
} dspark_sts_fit_args;

typedef struct dspark_sts_apply_args {
  uint32_t struct_size;
  int32_t R, gamma;
  const float* z;
  const float* tau;
  float* c;
  void* stream;
} dspark_sts_apply_args;

int dspark_sts_fit(const dspark_sts_fit_args* args);
int dspark_sts_apply(const dspark_sts_apply_args* args);

/* --------------------------------------------------------------------------
 * dspark_pack_w2: W2 rearranged once (at model load) into the layout the
 * 16-row fused bias kernel reads, so that each of its load instructions
 * reads 1 KiB contiguous instead of 64 bytes from each of 16 rows.
 *
 * For callers whose batches take the 16-row path (bf16 weights, R <= 64).
 * The packed copy holds the same weights as W2; passed as W2_packed to
 * dspark_draft_block and dspark_verify (which still need W2 itself for the
 * finish kernels' one-segment rescans), it is read instead of W2 by the
 * fused kernel.  It is not read on the other paths (R > 64, fp32 weights).
 *
 * Layout: KS = 2, 4, 8 or 16 for rank <= 64, 128, 256, 512; for segment
 * s = 0 .. ceil(V / 16) - 1 and k-step ks = 0 .. KS - 1, 64 slots of 8 bf16
 * (16 bytes) at byte offset ((s * KS + ks) * 64 + L) * 16, slot L = 16 q + i
 * holding W2[16 s + i][32 ks + 8 q .. 32 ks + 8 q + 7], zero where the row
 * is >= V or the column >= rank.
 *
 * Arguments:
 *   V, rank    host ints (as for dspark_draft_block; bf16 weights only).
 *   W2         bf16 [V, rank] device, 16-byte aligned.
 *   W2_packed  device, 16-byte aligned, dspark_w2_packed_bytes(V, rank)
 *              bytes, out; owned by the caller.
 *   stream     hipStream_t as void*.
 * -------------------------------------------------------------------------- */
typedef struct dspark_pack_w2_args {
  uint32_t struct_size;
  int32_t V, rank;
  const void* W2;
  void* W2_packed;
  size_t W2_packed_bytes;
  void* stream;
} dspark_pack_w2_args;

int dspark_pack_w2(const dspark_pack_w2_args* args);

/* Host-side: bytes of the packed W2 of dspark_pack_w2; 0 for an invalid
 * V or rank. */
size_t dspark_w2_packed_bytes(int32_t V, int32_t rank);

int dspark_draft_block(const dspark_draft_args* args);

/* --------------------------------------------------------------------------
 * dspark_draft_block_noalloc: dspark_draft_block for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, checks, kernels and results as dspark_draft_block, except
 * that `workspace` and `workspace_bytes` are ignored: the workspace is a
 * static device array of DSPARK_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device it runs on until the process ends (its address is
 * looked up once per device; nothing is allocated or freed by the call).  A
 * call whose dspark_draft_workspace_size() exceeds that size returns
 * DSPARK_ERR_WORKSPACE and enqueues nothing (64 MiB holds, e.g., R = 1024 at
 * V = 129280 with 64-row segments, or R <= 64 at V up to 2097136 with 16-row
 * segments and the Markov head; the RNN head's packed A takes
 * dspark_w2_packed_bytes(rank, rank) more).  DSPARK_CHECK_INPUTS is refused (DSPARK_ERR_UNSUPPORTED): the
 * checks report through a caller's workspace.  Every call on one device
 * shares the array, and a call leaves its contents behind: calls that
 * overlap in time on one device (another stream, another host thread) race
 * and must be serialised by the caller.
 * -------------------------------------------------------------------------- */
#define DSPARK_NOALLOC_SCRATCH_BYTES (64u << 20)
int dspark_draft_block_noalloc(const dspark_draft_args* args);
int dspark_schedule(const dspark_schedule_args* args);
int dspark_schedule_cutoff(const dspark_cutoff_args* args);
int dspark_verify(const dspark_verify_args* args);

/* Host-side: number of verify rows dspark_schedule emits,
 * R + min(max(K, 0), R * gamma); -1 for R < 0 or gamma < 1. */
int64_t dspark_schedule_rows(int32_t R, int32_t gamma, int64_t K);

/* Static description of a status code (never NULL). */
const char* dspark_status_string(int status);

/* DSPARK_ABI_VERSION of the loaded library. */
int dspark_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H_ */
