/*
 * rz.h -- C ABI of librz: batch-invariant per-token logprobs and the
 * REINFORCE Zero importance-sampling loss on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are cited by page title and section):
 *
 *  - log pi_theta(a_t | h_t): the learner's logprob of each sampled token,
 *    through a linear LM head (z = h W^T, W laid out [V, H], no bias,
 *    temperature 1), a log-softmax over the whole vocabulary and a gather.
 *    ("REINFORCE Zero" project page, section 02, "A minimal REINFORCE
 *    objective": pi_theta(a_it | h_it); the head itself is a reading, the
 *    pages never spell it out.)  The result for a row is bit-identical for
 *    the same (hidden row, W, token) whatever the number of rows, the row
 *    offset, the other rows in the batch or the entry point that computed
 *    it: the trainer-inference invariance the pages turn on (project page
 *    section 02 "Remove kernel mismatch"; vLLM blog "Zero mismatch, simple
 *    async RL", section 5, "diff 0").
 *
 *  - the unclipped token-level IS-REINFORCE loss (vLLM blog section 4, loss
 *    equation; project page "A minimal REINFORCE objective"):
 *        L = -(1/B) sum_i (1/T_i) sum_{valid t in i} A_i * w_t,
 *        w_t = exp(log pi_t - log mu_t)   (no clipping, no filtering),
 *        A_i = r_i - mean of r over the group of i,
 *        T_i = number of valid (mask = 1) rows of response i,
 *    and its gradient through the numerator pi_theta only, with respect to
 *    the hidden states and the LM-head weights.
 *
 *  - the diagnostics D3 = mean over valid tokens of (w - 1 - log w)
 *    (vLLM blog section 3) and the sampled rollout-to-learner KL, read as
 *    the k1 estimate mean(log mu - log pi) (vLLM blog section 4).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller, row-major
 *    and contiguous.  The library never allocates, frees or synchronises: it
 *    enqueues work on `stream` (NULL = the null stream) and
 *    outputs are valid once the stream reaches that point.
 *  - Scratch memory is a caller-provided device workspace of at least
 *    rz_workspace_bytes(...) or rz_workspace_bytes_op(...) bytes, 256-byte
 *    aligned.  Its contents on entry
 *    do not matter and on return are unspecified.
 *  - hidden and lm_head are fp32 (RZ_DTYPE_F32) or bfloat16 (RZ_DTYPE_BF16);
 *    every other floating-point array is fp32.  Arithmetic accumulates in
 *    fp32 (reductions over tokens in fp64).
 *  - Argument errors that the host can see return a negative rz_status
 *    before any HIP call (so they are testable without a GPU).  n_rows = 0
 *    is a valid no-op.
 *  - Errors only the device can see set bits in *err_flag (a device int32,
 *    may be NULL; bits are OR-ed in, never cleared) and turn the affected
 *    outputs into NaN; the call still completes normally.
 *  - The library keeps no state between calls except the optional kernel
 *    timer (rz_timing_*), which is kept per host thread: enabling it on one
 *    thread times only that thread's calls.
 */
#ifndef RZ_H_
#define RZ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared as the HIP runtime declares it, so that
 * this header needs no HIP header (repeating an identical typedef is legal
 * in C11 and C++). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  RZ_OK = 0,
  RZ_ERR_INVALID_ARG = -1, /* null required pointer, bad size or count     */
  RZ_ERR_UNSUPPORTED = -2, /* unknown dtype, H not a multiple of 64, ...    */
  RZ_ERR_WORKSPACE = -3,   /* workspace NULL, misaligned or too small      */
  RZ_ERR_HIP = -4,         /* a HIP launch or event call failed            */
  RZ_ERR_SCRATCH = -5      /* sizes need more than the static scratch of an
                              allocation-free entry point                   */
} rz_status;

typedef enum { RZ_DTYPE_F32 = 0, RZ_DTYPE_BF16 = 1 } rz_dtype;

typedef enum {
  RZ_OP_TOKEN_LOGPROBS = 0,
  RZ_OP_FWD_BWD = 1,
  RZ_OP_DIAGNOSTICS = 2,
  RZ_OP_SAMPLE = 3,
  RZ_OP_GRAD_NORMS = 4,
  RZ_OP_FWD_BWD_LORA = 5,
  RZ_OP_TOKEN_LOGPROBS_MX = 6,
  RZ_OP_SAMPLE_MX = 7,
  RZ_OP_SCORE_CENTERING = 8
} rz_op;

/* LoRA on the head: the largest rank, and the number of columns the
 * adapter adds to the augmented operands (columns past the rank hold 0). */
#define RZ_LORA_COLS 64

/* element format of an MX-format LM head (OCP Microscaling Formats v1.0) */
typedef enum {
  RZ_MX_FP4 = 0, /* MXFP4: E2M1 elements, two per byte (low nibble first) */
  RZ_MX_FP8 = 1  /* MXFP8: E4M3 elements, one per byte                     */
} rz_mx_format;

/* device-side error bits written to *err_flag */
#define RZ_DEVERR_TOKEN 1   /* a token id outside [0, V): its logprob is NaN  */
#define RZ_DEVERR_GROUP 2   /* a group id outside [0, n_resp): loss/adv NaN    */
#define RZ_DEVERR_CU_ROWS 4 /* cu_rows not 0..n_rows monotone: loss/adv NaN   */
#define RZ_DEVERR_MX_SCALE 8 /* an MX block scale outside the exact range     */

/* Alignment: every array the kernels move in 16-byte pieces -- hidden,
 * lm_head, d_hidden, d_lm_head, lora_A, the MX codes and scales, and the
 * gradient-norm inputs -- must start on a 16-byte boundary; an entry point
 * given one that does not returns RZ_ERR_INVALID_ARG before any HIP call. */

/* Limits checked on the host. */
#define RZ_MAX_ROWS ((int64_t)1 << 30)
#define RZ_MAX_VOCAB (1 << 24)
#define RZ_MAX_HIDDEN 32768
#define RZ_MAX_RESPONSES (1 << 24)

/* Bytes of workspace that rz_token_logprobs, rz_reinforce_zero_fwd_bwd and
 * rz_diagnostics need at these sizes: the largest of the three, so one
 * buffer serves all of them (n_resp is read by the learner step only; when
 * it is invalid the learner step's need is left out).  0 when the sizes are
 * invalid for all three. */
size_t rz_workspace_bytes(int64_t n_rows, int32_t n_resp, int32_t H,
                          int32_t V, rz_dtype dt);

/* Bytes of workspace one entry point needs (op names it); 0 when the sizes
 * are themselves invalid (the call would return an error anyway).  For
 * RZ_OP_DIAGNOSTICS only n_rows is read; for RZ_OP_GRAD_NORMS, n_rows, H and
 * V (dt is ignored).  rz_response_diagnostics and rz_run_summary need no
 * workspace. */
size_t rz_workspace_bytes_op(rz_op op, int64_t n_rows, int32_t n_resp,
                             int32_t H, int32_t V, rz_dtype dt);

/* Static description of an error code. Never NULL. */
const char* rz_status_string(rz_status s);

/*
 * rz_token_logprobs -- the rollout-shaped (or learner-shaped) forward.
 *
 *   hidden   [n_rows, H]  dt      final hidden state of each history h_t
 *   lm_head  [V, H]       dt      LM-head weights W
 *   tokens   [n_rows]     int32   sampled token a_t of each row
 *   logprobs [n_rows]     fp32    out: log pi(a_t | h_t)
 *   lse      [n_rows]     fp32    out, may be NULL: log sum_v exp(z[t, v])
 *   err_flag              int32   may be NULL; RZ_DEVERR_TOKEN on bad tokens
 *
 * H must be a multiple of 64.  Rows are independent; the row's result does
 * not depend on n_rows, on its position or on the other rows.
 */
rz_status rz_token_logprobs(const void* hidden, const void* lm_head,
                            const int32_t* tokens, int64_t n_rows, int32_t H,
                            int32_t V, rz_dtype dt, float* logprobs,
                            float* lse, int32_t* err_flag, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * rz_reinforce_zero_fwd_bwd -- one learner step of the hot path.
 *
 *   hidden    [n_rows, H]  dt     final hidden states, responses packed
 *   lm_head   [V, H]       dt     LM-head weights
 *   tokens    [n_rows]     int32  sampled tokens (the caller has applied the
 *                                 next-token shift: row t predicts tokens[t])
 *   logmu     [n_rows]     fp32   recorded behaviour logprob log mu of tokens[t]
 *   mask      [n_rows]     uint8  1 = valid action token, 0 = masked row
 *   cu_rows   [n_resp + 1] int32  response i owns rows [cu_rows[i], cu_rows[i+1]);
 *                                 cu_rows[0] = 0, cu_rows[n_resp] = n_rows
 *   rewards   [n_resp]     fp32   scalar reward r_i
 *   group_ids [n_resp]     int32  group of response i, in [0, n_resp)
 *
 *   logprobs  [n_rows]     fp32 out: log pi on valid rows, 0 on masked rows
 *   loss      [1]          fp32 out: L (above)
 *   d_hidden  [n_rows, H]  fp32 out: dL/dhidden; zero rows where mask = 0
 *   d_lm_head [V, H]       fp32 out: dL/dW, overwritten (not accumulated)
 *   diag      [2]          fp32 out, may be NULL: {D3, KL} over valid rows,
 *                               bit-identical to rz_diagnostics(logprobs,
 *                               logmu, mask) on this call's outputs
 *   adv       [n_resp]     fp32 out, may be NULL: A_i
 *
 * A response with T_i = 0 adds nothing to L or the gradients; B = n_resp
 * still counts it.  No clipping is applied anywhere: a large log-ratio gives
 * an infinite weight and loss, as the method prescribes.
 * Device-detected faults: RZ_DEVERR_TOKEN (that row's logprob is NaN, and so
 * are the loss and gradients it feeds), RZ_DEVERR_GROUP and RZ_DEVERR_CU_ROWS
 * (loss, adv and the gradients are NaN).
 * Determinism: every output is identical run to run for identical inputs;
 * logprobs rows are additionally batch-invariant as in rz_token_logprobs.
 */
rz_status rz_reinforce_zero_fwd_bwd(
    const void* hidden, const void* lm_head, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lm_head, float* diag, float* adv,
    int32_t* err_flag, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rz_score_centering_fwd_bwd -- the score-centering (SC) update: the same
 * learner step without importance weights.
 *
 * "REINFORCE Zero" project page, "The full IS correction", blocks 02-03:
 * sampled under q, the plain update E_q[A s] is the covariance Cov_q(A, s)
 * plus the drift E_q[A] E_q[s]; SC removes the drift and keeps
 * g_SC = Cov_q(A, s) = E_q[(A - E_q A) s].  The group-mean advantage A_i is
 * that centred factor, so the estimate is the unclipped IS loss's gradient
 * with w replaced by 1 (vLLM blog, section 4 "Results", runs "Score
 * Centering without IS" as a training arm).  This call computes
 *     L_SC = -(1/B) sum_i (1/T_i) sum_{valid t in i} A_i log pi_t,
 *     c_t  = A_i / (B T_i)   (minus dL_SC / d log pi_t),
 * and dL_SC/dhidden, dL_SC/dW through log pi, on the kernels of
 * rz_reinforce_zero_fwd_bwd (only c_t and the loss's per-token term
 * differ).  Arguments and outputs as rz_reinforce_zero_fwd_bwd, except:
 *   logmu  may be NULL (SC never reads it); then diag must be NULL.  With
 *          logmu given, diag is {D3, KL} of the rollout records, as in
 *          rz_reinforce_zero_fwd_bwd.
 *   loss   L_SC above (its gradient is the SC update, negated).
 * logprobs are bit-identical to rz_reinforce_zero_fwd_bwd's.  Workspace:
 * rz_workspace_bytes(n_rows, n_resp, H, V, dt) (RZ_OP_SCORE_CENTERING).
 */
rz_status rz_score_centering_fwd_bwd(
    const void* hidden, const void* lm_head, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lm_head, float* diag, float* adv,
    int32_t* err_flag, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * rz_sample_tokens -- the rollout side: draw each row's token and record
 * its logprob ("Zero mismatch, simple async RL", vLLM blog, section 4
 * "Recipe" item 2: the rollout records the logprob of every token it
 * samples; section 5: "diff 0", rollout and trainer compute bit-identical
 * logprobs for every sampled token).
 *
 *   hidden   [n_rows, H]  dt      final hidden state of each history h_t
 *   lm_head  [V, H]       dt      LM-head weights W
 *   row_ids  [n_rows]     uint64  a caller-chosen identity of each row
 *   seed                  uint64  key of the draw
 *   tokens   [n_rows]     int32   out: a_t
 *   logmu    [n_rows]     fp32    out: log pi(a_t | h_t), the record
 *   lse      [n_rows]     fp32    out, may be NULL: log sum_v exp(z[t, v])
 *
 * The draw is from softmax(z_t) at temperature 1 by the Gumbel-max rule:
 * a_t = argmax_v z[t, v] - log(-log u[t, v]), ties to the smaller v, with
 * u = (x + 1/2) 2^-32 and x = word v % 4 of Philox4x32-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) at counter
 * (v / 4, id low word, id high word, 0) and key (seed low word, seed high
 * word).  A row's token depends on (seed, its id, hidden, W) only, not on
 * n_rows or the other rows.  logmu and lse are computed by the kernels of
 * rz_token_logprobs, so logmu is bit-identical to rz_token_logprobs(hidden,
 * lm_head, tokens) at the same weights.  H must be a multiple of 64.
 */
rz_status rz_sample_tokens(const void* hidden, const void* lm_head,
                           const uint64_t* row_ids, int64_t n_rows, int32_t H,
                           int32_t V, rz_dtype dt, uint64_t seed,
                           int32_t* tokens, float* logmu, float* lse,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Bytes of the static device scratch of rz_sample_tokens_noalloc, per GPU. */
#define RZ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * rz_sample_tokens_noalloc -- rz_sample_tokens for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments and outputs as
 * rz_sample_tokens, without the workspace: the draw's scratch (the
 * statistics-tile partials and the draw candidates with their logits;
 * rz_workspace_bytes_op(RZ_OP_SAMPLE, n_rows, 1, H, V, dt) bytes) lives in
 * a static device array of RZ_NOALLOC_SCRATCH_BYTES on each GPU, which the
 * library holds from its first use on that GPU until the process ends.
 * Sizes that need more return RZ_ERR_SCRATCH before any HIP call (at
 * V = 151936, more than about 2800 rows).  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine) and its outputs are
 * those of rz_sample_tokens bit for bit (the same kernels).  Every call on
 * a GPU uses that GPU's one array: calls that may overlap on one GPU (other
 * streams, other host threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs to start at zero.
 */
rz_status rz_sample_tokens_noalloc(const void* hidden, const void* lm_head,
                                   const uint64_t* row_ids, int64_t n_rows,
                                   int32_t H, int32_t V, rz_dtype dt,
                                   uint64_t seed, int32_t* tokens, float* logmu,
                                   float* lse, hipStream_t stream);

/*
 * rz_diagnostics -- D3 and the k1 rollout-to-learner KL.
 *
 *   logpi [n] fp32, logmu [n] fp32, mask [n] uint8 (may be NULL = all valid)
 *   diag  [2] fp32 out: {mean(expm1(d) - d), mean(-d)} over valid entries,
 *         d = logpi - logmu; NaN for both when no entry is valid.
 *
 * The reduction order depends only on n, so the result is a pure function
 * of (logpi, logmu, mask, n).
 */
rz_status rz_diagnostics(const float* logpi, const float* logmu,
                         const uint8_t* mask, int64_t n, float* diag,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * rz_dequantize_head -- an LM head stored at release precision, as MX
 * blocks, expanded to the bfloat16 head every other entry point takes
 * ("Zero mismatch, simple async RL", vLLM blog: the aligned path keeps
 * release precision, FP8 and MXFP4 weights included, with zero mismatch
 * between rollout and trainer).
 *
 *   codes   RZ_MX_FP4: [V, H / 2] bytes, element 2j of a row in the low
 *           nibble of byte j; RZ_MX_FP8: [V, H] bytes (device, 16-byte aligned)
 *   scales  [V, H / 32] E8M0 bytes: block b of row v covers elements
 *           32 b .. 32 b + 31 and scales them by 2^(scales[v, b] - 127)
 *   lm_head [V, H] bf16 out (device, 16-byte aligned)
 *   err_flag int32, may be NULL: RZ_DEVERR_MX_SCALE is or-ed in when a block
 *           scale is the NaN code 255 or outside the exact range below
 *
 * Element values follow the OCP Microscaling Formats v1.0 encodings (E2M1:
 * bias 1, largest 6; E4M3: bias 7, largest 448, S.1111.111 NaN).  With scale
 * 2^s every value of a block is exactly a bfloat16 number when s <= 125
 * (E2M1) or -124 <= s <= 119 (E4M3); such blocks are converted with no
 * rounding, so running the bf16 entry points on the output is the MX head
 * itself, and rollout and learner calls on it agree bit for bit.  Blocks
 * outside the range are written as NaN; an E4M3 NaN code gives a NaN value.
 * H must be a multiple of 32 (the GEMM entry points need 64).  No workspace.
 */
rz_status rz_dequantize_head(const uint8_t* codes, const uint8_t* scales,
                             int32_t V, int32_t H, rz_mx_format fmt,
                             void* lm_head, int32_t* err_flag, hipStream_t stream);

/*
 * rz_token_logprobs_mx, rz_sample_tokens_mx -- rz_token_logprobs and
 * rz_sample_tokens on a head stored as MX blocks (codes and scales as in
 * rz_dequantize_head; 16-byte aligned), with bf16 hidden states.
 *
 * Their results are bit-identical to the bf16 calls on
 * rz_dequantize_head(codes, scales), the expanded head, in every case (same
 * MFMA operands, same folds).  Up to 128 rows (rz_token_logprobs_mx) or 256
 * rows (rz_sample_tokens_mx), and with H a multiple of 128, the 64-row tile
 * reads the codes directly: a quarter (MXFP4) or a half (MXFP8) of the bf16
 * head's bytes per call, which is what bounds the rollout at decode size.
 * Otherwise the head is expanded into the workspace first.  Blocks with an
 * invalid scale give NaN and set RZ_DEVERR_MX_SCALE in err_flag (may be
 * NULL).  Workspace: rz_workspace_bytes_op(RZ_OP_TOKEN_LOGPROBS_MX or
 * RZ_OP_SAMPLE_MX, n_rows, 1, H, V, RZ_DTYPE_BF16).
 */
rz_status rz_token_logprobs_mx(const void* hidden, const uint8_t* codes,
                               const uint8_t* scales, rz_mx_format fmt,
                               const int32_t* tokens, int64_t n_rows, int32_t H,
                               int32_t V, float* logprobs, float* lse,
                               int32_t* err_flag, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
rz_status rz_sample_tokens_mx(const void* hidden, const uint8_t* codes,
                              const uint8_t* scales, rz_mx_format fmt,
                              const uint64_t* row_ids, int64_t n_rows,
                              int32_t H, int32_t V, uint64_t seed,
                              int32_t* tokens, float* logmu, float* lse,
                              int32_t* err_flag, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * LoRA adapter on the head ("Zero mismatch, simple async RL", vLLM blog,
 * Kimi K3.1 section: zero mismatch holds with LoRA adapters on every module
 * and through LoRA training; LoRA as in Hu et al., 2021).
 *
 * The adapted head is z = h W^T + u B^T with u = scale * (h A^T) rounded to
 * the head's precision (nearest bf16, ties to even, for RZ_DTYPE_BF16; fp32
 * for RZ_DTYPE_F32): the plain head over the augmented operands
 * h_aug = [h | u | 0] [n, H + RZ_LORA_COLS] and W_aug = [W | B | 0]
 * [V, H + RZ_LORA_COLS].  The rollout builds them with the two calls below
 * (the head once per weight update) and runs rz_token_logprobs /
 * rz_sample_tokens on them with H + RZ_LORA_COLS as the hidden size; the
 * learner's rz_reinforce_zero_fwd_bwd_lora builds the same operands with the
 * same kernels, so rollout records and learner logprobs agree bit for bit.
 * u is computed by the GEMM tile engine in a fixed K order, so a row's u
 * does not depend on the batch.
 *
 *   lora_A [r, H] dt, lora_B [V, r] dt (device), 1 <= r <= RZ_LORA_COLS,
 *   scale the adapter's scale (alpha / r); H a multiple of 64 with
 *   H + RZ_LORA_COLS <= RZ_MAX_HIDDEN.
 *
 * rz_lora_augment:    hidden_aug [n_rows, H + RZ_LORA_COLS] dt out.
 * rz_lora_merge_head: head_aug [V, H + RZ_LORA_COLS] dt out.
 * Neither takes a workspace.
 */
rz_status rz_lora_augment(const void* hidden, const void* lora_A, float scale,
                          int64_t n_rows, int32_t H, int32_t r, rz_dtype dt,
                          void* hidden_aug, hipStream_t stream);
rz_status rz_lora_merge_head(const void* lm_head, const void* lora_B,
                             int32_t V, int32_t H, int32_t r, rz_dtype dt,
                             void* head_aug, hipStream_t stream);

/*
 * rz_reinforce_zero_fwd_bwd_lora -- the learner step with a LoRA adapter on
 * a frozen head.  Arguments as rz_reinforce_zero_fwd_bwd, plus lora_A,
 * lora_B, scale and r as above; outputs:
 *
 *   logprobs, loss, diag, adv   as rz_reinforce_zero_fwd_bwd (log pi of the
 *                               adapted head; bit-identical to
 *                               rz_token_logprobs on the augmented operands)
 *   d_hidden  [n_rows, H] fp32  dL/dh through W and through the adapter
 *   d_lora_A  [r, H] fp32       dL/dA = scale (dL/du)^T h
 *   d_lora_B  [V, r] fp32       dL/dB = (dL/dz)^T u
 *
 * The rounding of u is treated as the identity in the backward pass.  W gets
 * no gradient and none is computed.  dL/dA sums fixed chunks of 4096 rows in
 * order.  Workspace: rz_workspace_bytes_op(RZ_OP_FWD_BWD_LORA, n_rows,
 * n_resp, H, V, dt) (independent of r).
 */
rz_status rz_reinforce_zero_fwd_bwd_lora(
    const void* hidden, const void* lm_head, const void* lora_A,
    const void* lora_B, float scale, int32_t r, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lora_A, float* d_lora_B,
    float* diag, float* adv, int32_t* err_flag, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Run-level diagnostics ("Zero mismatch, simple async RL", vLLM blog,
 * section 3 and Figure 1: the per-update D3 over a run, its peak against its
 * median; section 4 "What happens without alignment": the median
 * rollout-to-learner KL over the first and the last 1,000 updates and the
 * largest gradient norm before clipping.  "REINFORCE Zero" project page,
 * section 01, Figure 2: batch-averaged D3, peak over median.)
 *
 * rz_grad_norms -- L2 norms of this path's two gradients.
 *
 *   d_hidden  [n_rows, H] fp32  dL/dhidden (device, 16-byte aligned; may be
 *                               NULL when n_rows = 0)
 *   d_lm_head [V, H]      fp32  dL/dW (device, 16-byte aligned)
 *   norms     [2]         fp32  out (device): {||d_hidden||_2, ||d_lm_head||_2}
 *
 * Sums of squares are taken in float64 over fixed chunks of 65536 values
 * and then over the chunks in a fixed tree, so the result is a pure
 * function of the inputs and their sizes.  Workspace:
 * rz_workspace_bytes_op(RZ_OP_GRAD_NORMS, n_rows, 0, H, V, 0).
 */
rz_status rz_grad_norms(const float* d_hidden, int64_t n_rows, int32_t H,
                        const float* d_lm_head, int32_t V, float* norms,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rz_response_diagnostics -- D3 and KL of each response (rz_diagnostics
 * restricted to one response's valid rows).
 *
 *   logpi, logmu [n_rows] fp32, mask [n_rows] uint8 (may be NULL = all
 *   valid), cu_rows [n_resp + 1] int32 as in rz_reinforce_zero_fwd_bwd
 *   (all device).
 *   d3, kl [n_resp] fp32 out (device): mean(expm1(d) - d) and mean(-d) over
 *   response i's valid rows, d = logpi - logmu, accumulated in float64 in a
 *   fixed order; NaN for a response with no valid row.
 *   err_flag int32, may be NULL: RZ_DEVERR_CU_ROWS is or-ed in when a
 *   response's range is not an ordered range inside [0, n_rows), or
 *   cu_rows[0] != 0 or cu_rows[n_resp] != n_rows; such responses read NaN.
 *
 * No workspace.  n_resp = 0 is a no-op.
 */
rz_status rz_response_diagnostics(const float* logpi, const float* logmu,
                                  const uint8_t* mask, const int32_t* cu_rows,
                                  int64_t n_rows, int32_t n_resp, float* d3,
                                  float* kl, int32_t* err_flag, hipStream_t stream);

/*
 * rz_run_summary -- the run-level view over per-step records (host memory,
 * host code; no GPU work).
 *
 *   d3, kl, grad_norm [n_steps] fp32 host arrays of per-step values in
 *   step order; any may be NULL, which makes its outputs NaN.
 *   window            steps in each KL window (>= 1; a run shorter than
 *                     the window uses all its steps for both).
 *   out [7] float64 host: {D3 peak, D3 median, D3 peak / median, median KL
 *   over the first `window` steps, median KL over the last `window` steps,
 *   last / first, largest gradient norm}.
 *
 * The median of an even count is the mean of the two middle values.  An
 * array holding a NaN gives NaN for its statistics; quotients follow IEEE
 * division (a zero median, as in a run with D3 = 0 at every step, gives
 * inf or NaN).  n_steps = 0 gives NaN throughout.
 */
rz_status rz_run_summary(const float* d3, const float* kl,
                         const float* grad_norm, int64_t n_steps,
                         int32_t window, double* out);

/*
 * Kernel timer (measurement support).  While enabled, every kernel launch of
 * the entry points above is bracketed by a pair of HIP events on the call's
 * stream.  rz_timing_read waits for those events, adds each launch's elapsed
 * time to its kernel's total, and copies totals (milliseconds) and launch
 * counts for kernels 0 .. rz_timing_num_kernels()-1; reset != 0 clears them.
 * Enabling creates the events (host-side driver objects, no device memory);
 * disabling destroys them.  The timer's state is per host thread.
 */
rz_status rz_timing_enable(int on);
int rz_timing_num_kernels(void);
const char* rz_timing_kernel_name(int k);
rz_status rz_timing_read(double* total_ms, int64_t* launches, int reset);

/*
 * Matrix-core ceiling (measurement support, not part of the method).
 * rz_calibrate_mfma launches n_workgroups workgroups of four waves (one per
 * SIMD; each SIMD gets the MFMA stream of the GEMM tile's two waves on it,
 * 128 x 128 accumulators); each wave issues iters x 128 MFMAs of the
 * learner GEMMs' instruction (v_mfma_f32_32x32x16_bf16, 32768 FLOP each)
 * into sixteen 32 x 32 accumulators, with operands kept in registers
 * (from_lds = 0) or read from LDS before every sixteen MFMAs, as the GEMM
 * reads them (from_lds = 1), and no global memory traffic.  data = 1 gives
 * the operands random-looking bf16 values, data = 0 all zeros.  FLOP per
 * launch: n_workgroups x 4 x iters x 128 x 32768.  sink [n_workgroups x 256]
 * fp32 (device) receives the accumulator sums.  Timed by the caller (HIP
 * events on `stream`); rocprofv3 counters of the launch give the clock and
 * the matrix cores' busy share.
 */
rz_status rz_calibrate_mfma(int32_t data, int32_t from_lds, int32_t n_workgroups,
                            int64_t iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RZ_H_ */
