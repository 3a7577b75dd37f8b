/*
 * domino_head.h -- C ABI of the MI355X (gfx950) Domino head drafting library.
 *
 * The Domino head (paper.oopus.info review of "Domino: Decoupling Causal
 * Modeling from Autoregressive Drafting in Speculative Decoding", section 二,
 * 第二步 Domino Head) turns the output of a parallel draft backbone -- hidden
 * states H and base logits L_base for a whole block, produced in one forward
 * pass (same section, 第一步; news.sig.ai article, section "Domino怎么做") --
 * into a causally consistent greedy draft.  For block positions p = 0..K-1:
 *
 *     u_p       = SiLU(W1 [H_p ; S_p])                    (rank r, no bias)
 *     L_final_p = L_base_p + W2 u_p                        (logit space)
 *     t_p       = argmax_v L_final_p[v]                    (greedy decoding)
 *     S_{p+1}   = GRU(E[x_p], S_p),  x_p = t_p or teacher[p]
 *
 * with S_0 = GRU(E[last_tok], S_init) (anchor step on the last confirmed
 * token; S_init = 0 when not given).  GRU is PyTorch's GRUCell: rows of
 * W_ih/W_hh/b_ih/b_hh in blocks (reset, update, new);
 *     r = sig(W_ir x + b_ir + W_hr s + b_hr), z = sig(W_iz x + b_iz + W_hz s + b_hz),
 *     n = tanh(W_in x + b_in + r * (W_hn s + b_hn)),  s' = (1 - z) * n + z * s.
 * SiLU(a) = a * sig(a).  Ties in the argmax go to the lowest index; a NaN
 * logit counts as larger than any number (the first NaN wins); -0 equals +0.
 * The head state S and all accumulation are float32.
 *
 * Every entry point returns 0 on success or a negative DOMINO_E* code; the
 * message of the last failure on the calling thread is domino_last_error().
 * Device work is asynchronous and ordered on the given HIP stream (NULL =
 * the null stream); nothing synchronizes except domino_head_check_error.
 * All tensors are row-major and contiguous, owned by the caller, and every
 * device pointer must be 16-byte aligned.
 */
#ifndef DOMINO_HEAD_H
#define DOMINO_HEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ---- */
#define DOMINO_OK 0
#define DOMINO_EINVAL (-1)      /* bad argument: NULL, misaligned, B out of range, K > 16 */
#define DOMINO_EUNSUPPORTED (-2) /* dimensions or dtype the kernels do not handle */
#define DOMINO_EWORKSPACE (-3)  /* workspace missing or smaller than domino_head_workspace_size */
#define DOMINO_EHIP (-4)        /* a HIP runtime call failed (message carries the HIP error) */
#define DOMINO_EDEVICE (-5)     /* domino_head_check_error found device-side flags */

/* ---- weight storage types ---- */
#define DOMINO_F32 0
#define DOMINO_BF16 1

/* ---- device-side flags reported by domino_head_check_error ---- */
#define DOMINO_FLAG_BAD_TOKEN 1u      /* a last_tok or used teacher id was outside [0, V) */
#define DOMINO_FLAG_SYNC_TIMEOUT 2u   /* a grid barrier spin limit ran out; outputs invalid */

/* ---- config.flags bits (execution strategy).  For B <= 8 every launch gives the same bits; for
 * B > 8 the launches round u to one bf16 matrix-core operand and agree with each other up to the
 * order of float32 sums (the logits move by at most about 1e-2 against the oracle either way) ---- */
#define DOMINO_EXEC_AUTO 0u        /* pick per call from B: the persistent launch for B <= 8, and for
                                      8 < B <= 256 where the batched persistent launch is available (see
                                      below); the step launches otherwise */
#define DOMINO_EXEC_PERSISTENT 1u  /* one cooperative launch covering all K positions: B <= 8, or (bf16
                                      weights, r = 256, DOMINO_FOLD_EMBED or DOMINO_MARKOV, h a multiple
                                      of 64, d of 32) B <= 256, where the GRU update and state products
                                      (for a Markov head, the table gather that forms u) are spread over
                                      the grid; either way each block keeps its W2 slice on chip */
#define DOMINO_EXEC_STEPWISE 2u    /* one launch per phase and position */
#define DOMINO_EXEC_STREAM_W2 8u   /* persistent launch: stream W2 from memory at every position instead of
                                      keeping the slice on chip (bf16, r = 256); for comparison */
#define DOMINO_FOLD_EMBED 4u       /* precompute P = E W_ih^T + b_ih ([V, 3h] float32, in the workspace) at
                                      create time, so each GRU step gathers one row of P instead of
                                      multiplying W_ih by the embedding row (same values up to rounding) */
#define DOMINO_EXEC_PLAIN_LAUNCH 16u /* persistent launch as an ordinary kernel launch instead of a
                                      cooperative one (about 17 us less dispatch time per call).  Its
                                      blocks (one per compute unit) wait for each other, so the caller
                                      guarantees that no other kernel that waits for other work (in
                                      particular no other persistent draft) runs on the device at the
                                      same time; otherwise the bounded waits time out and the call
                                      reports DOMINO_FLAG_SYNC_TIMEOUT.  A process that needs the
                                      persistent launch while another process that has made
                                      cooperative launches on the same GPU is alive sets this flag:
                                      the HIP runtime refuses that second process's cooperative
                                      launches (the draft returns DOMINO_EHIP, "the operation cannot
                                      be performed in the present state") */

#define DOMINO_EXEC_POSITION_BATCHED 32u /* with a teacher: take the step launches even for B <= 8.  With
                                      a teacher the states of all positions follow from the given
                                      tokens alone, so the step launches run the GRU chain first and
                                      then the W2 products of all K positions as one launch over B*K
                                      rows (W2 read once instead of K times); they always do this
                                      when a teacher is given.  Same values as the per-position
                                      launches, bit for bit */

#define DOMINO_LBASE_BF16 64u         /* domino_head_draft's L_base holds bfloat16 bit patterns instead of
                                      float32: half the bytes of the base-logit stream, which dominates
                                      at large B.  Every path widens each value exactly, so the draft
                                      equals a float32 call on the widened values bit for bit */

/* ---- config.flags bit that changes the model ---- */
#define DOMINO_MARKOV 128u            /* Markov head instead of the recurrent one.  The news.sig.ai
                                      article (section 从Domino看DSpark) names a Markov head, DSpark's
                                      default, beside an RNN head that corresponds to Domino's causal
                                      encoder, and gives no formula.  Reading taken: each position is
                                      conditioned on the token before it alone, S_p = GRU(E[x_p], 0)
                                      with x_0 = last_tok and x_p = t_{p-1} (or teacher[p-1]), so
                                      W1_S S_p is a row of the per-token table M = W1_S GRU(E[t], 0)
                                      ([V, r] float32 in the workspace, filled at create) and
                                      u_p = SiLU(W1_H H_p + M[x_p]).  The same weights serve both
                                      heads.  Not combinable with DOMINO_FOLD_EMBED or
                                      DOMINO_EXEC_STREAM_W2; domino_head_draft then takes no S_init
                                      and writes no S_out (both must be NULL) */

/*
 * Head configuration.  All weight pointers are DEVICE pointers, borrowed for
 * the lifetime of the handle (never copied, never written), stored in
 * `wdtype` (float32, or bfloat16 as raw 16-bit patterns):
 *   W1   [r, d+h]  columns 0..d-1 multiply H_p, columns d..d+h-1 multiply S_p
 *   W2   [V, r]
 *   W_ih [3h, d], W_hh [3h, h]   GRU weights, row blocks (reset, update, new)
 *   b_ih [3h], b_hh [3h]         GRU biases, NULL means zero
 *   E    [V, d]                  token embedding table (the GRU input rows)
 * Limits: 1 <= K <= 16; d, h multiples of 8, h <= 2048; r/8 (bf16) or r/4
 * (float32) a power of two, r <= 1024; 1 <= max_batch <= 1024; V >= 1.
 */
typedef struct domino_head_config {
    int32_t d, h, r, V, K, max_batch;
    int32_t wdtype;
    uint32_t flags;
    const void *W1, *W2, *W_ih, *W_hh, *b_ih, *b_hh, *E;
} domino_head_config;

typedef struct domino_head *domino_head_t;

/* Host only.  Bytes of device workspace a handle with this config needs. */
int domino_head_workspace_size(const domino_head_config *cfg, size_t *bytes);

/*
 * Validates cfg and binds the caller-allocated device `workspace` (>=
 * domino_head_workspace_size bytes, 256-byte aligned, not shared with another
 * handle).  No allocation.  Without DOMINO_FOLD_EMBED or DOMINO_MARKOV no
 * device work either; with one of them, kernels fill the folded table (or the
 * Markov table, in chunks of tokens through a create-time region of the
 * workspace) on the null stream and create
 * waits for it.  On success *out is a new handle; release it with
 * domino_head_destroy.  The workspace state is cleared by the first draft.
 */
int domino_head_create(const domino_head_config *cfg, void *workspace, size_t workspace_bytes,
                       domino_head_t *out);

/*
 * Draft one block for B rows (1 <= B <= max_batch).  Device pointers:
 *   H        [B, K, d]  wdtype     backbone hidden states of the block
 *   L_base   [B, K, V]  float32    backbone base logits of the block (bfloat16
 *                                  bit patterns with DOMINO_LBASE_BF16)
 *   last_tok [B]        int32      last confirmed token (anchor GRU input)
 *   teacher  [B, K]     int32      NULL = free running; else teacher forcing:
 *                                  teacher[b][p] replaces t_p as GRU input for
 *                                  p <= K-2 (teacher[b][K-1] is never read)
 *   S_init   [B, h]     float32    NULL = zero initial state
 * Outputs (device):
 *   tokens   [B, K]     int32      greedy draft t_0..t_{K-1}; -1 for every
 *                                  position of a row whose last_tok or used
 *                                  teacher id lies outside [0, V)
 *   L_final  [B, K, V]  float32    NULL = not stored
 *   S_out    [B, K, h]  float32    NULL = not stored; S_0..S_{K-1}
 *   u_out    [B, K, r]  float32    NULL = not stored; u_0..u_{K-1}
 * Outputs may not alias inputs.  One draft may be in flight per handle (the
 * workspace is reused); calls on one handle must be ordered on one stream.
 * Bad token ids and barrier timeouts never abort: they set device flags read
 * by domino_head_check_error.
 */
int domino_head_draft(domino_head_t hd, int32_t B, const void *H, const void *L_base, const int32_t *last_tok,
                      const int32_t *teacher, const float *S_init, int32_t *tokens, float *L_final, float *S_out,
                      float *u_out, void *stream);

/*
 * Verify-side accept length (paper.oopus.info review, section 一; the
 * researchpapers.dev summary, 关键结果: the verifier keeps the longest draft
 * prefix that equals its own tokens).  Device pointers: draft, target [B, K]
 * int32; out_len [B] int32 receives the first p with draft[b][p] !=
 * target[b][p], or K when the whole row matches.  0 <= B, 1 <= K <= 16;
 * B = 0 is a no-op.  Raw int32 comparison, asynchronous on `stream`.
 */
int domino_accept_len(int32_t B, int32_t K, const int32_t *draft, const int32_t *target, int32_t *out_len,
                      void *stream);

/*
 * Greedy verify step of speculative decoding (paper.oopus.info review, section
 * 一: the target model checks the whole drafted block in one parallel pass and
 * keeps what it would have produced itself; researchpapers.dev summary, 关键结果
 * and 常见问题: every accepted token is the target's own).  Device pointers:
 *   logits   [B, K+1, V] float32  target logits; row j scores the token after
 *                                 the context plus draft[b][0..j-1], row K
 *                                 follows the whole draft
 *   draft    [B, K] int32         the drafted block (e.g. domino_head_draft's
 *                                 tokens; -1 entries simply never match)
 *   workspace                     >= domino_verify_workspace_size(B, K, V) bytes,
 *                                 scratch for this call (contents need no
 *                                 initialisation and are not read afterwards)
 * Outputs (device):
 *   target   [B, K+1] int32       NULL = not stored; argmax of each row, with
 *                                 the draft's rules (lowest index on ties, a
 *                                 NaN above every number, -0 == +0)
 *   accept   [B] int32            first j < K with draft[b][j] != target[b][j],
 *                                 else K
 *   next     [B] int32            target[b][accept[b]]: the target's token after
 *                                 the accepted prefix; the step commits
 *                                 draft[b][0..accept-1] and then this token,
 *                                 which is the next block's last_tok
 * 0 <= B; 1 <= K <= 16; V >= 1.  B = 0 is a no-op.  All pointers 16-byte
 * aligned; outputs may not alias inputs or the workspace.  Two kernel launches,
 * asynchronous on `stream`; no allocation, no synchronization.
 */
int domino_verify_workspace_size(int32_t B, int32_t K, int32_t V, size_t *bytes);
int domino_verify(int32_t B, int32_t K, int32_t V, const float *logits, const int32_t *draft, void *workspace,
                  size_t workspace_bytes, int32_t *target, int32_t *accept, int32_t *next, void *stream);

/*
 * domino_verify without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, outputs and results as domino_verify
 * (same kernels), but the per-call scratch (one 8-byte key per (row, chunk))
 * lives in a 1 MiB static device array of the library, one per device, held
 * until the process ends.  Nothing is allocated and nothing needs clearing
 * (every scratch word a call reads it has written first).  Returns
 * DOMINO_EUNSUPPORTED, before any device work, when
 * domino_verify_workspace_size(B, K, V) exceeds 1 MiB (about B (K+1) + 2048 >
 * 131072).  All calls on one device share the array: calls that may overlap
 * on one device (different streams, or host threads) race and give wrong
 * results; order them on one stream.
 */
int domino_verify_noalloc(int32_t B, int32_t K, int32_t V, const float *logits, const int32_t *draft,
                          int32_t *target, int32_t *accept, int32_t *next, void *stream);

/*
 * Synchronizes the device (every stream, so drafts replayed from a captured
 * HIP graph on any stream are included), reads and clears the device flags
 * (DOMINO_FLAG_*) into *device_flags (may be NULL) and resets the handle's
 * barrier state (the next draft clears it on the device before it runs).
 * Returns DOMINO_EDEVICE if any flag was set.
 */
int domino_head_check_error(domino_head_t hd, uint32_t *device_flags);

/*
 * Host only, no device work.  Which launch domino_head_draft takes for B rows
 * on this handle: *persistent = 1 for the single cooperative launch that runs
 * the whole drafting loop, 0 for one launch per step; *w2_resident = 1 when
 * that persistent launch keeps each block's share of W2 on chip across the K
 * positions instead of re-reading it; *grid = blocks of the persistent launch
 * (0 for the per-step launches).  Output pointers may be NULL.  Same errors as
 * domino_head_draft for B and for a forced persistent launch that cannot run.
 */
int domino_head_exec_info(domino_head_t hd, int32_t B, int32_t *persistent, int32_t *w2_resident, int32_t *grid);

/*
 * Host only.  Bound on every device-side wait of later drafts on this handle
 * (grid barriers, argmax and operand arrivals), in polling iterations of
 * roughly 0.1-1 us each.  A wait that runs out sets DOMINO_FLAG_SYNC_TIMEOUT
 * and its block leaves the launch, so every launch ends even if a block never
 * arrives.  The default is 2^22 (or DOMINO_BARRIER_SPIN_LIMIT from the
 * environment at create); 0 makes every wait give up at once, which forces
 * the timeout path from the host.
 */
int domino_head_set_spin_limit(domino_head_t hd, uint32_t limit);

/*
 * Host only.  Parameters of the head: r(d+h) + V r + 3h d + 3h h (+ 6h if GRU
 * biases are given); the embedding table E is the target's and not counted.
 * The paper.oopus.info review (section 二, 第二步 Domino Head) puts the head at
 * about 56 million parameters, 5.3% of the drafter: 55,934,976 (+6,144 biases)
 * at d = 4096, h = 1024, r = 256, V = 151936.
 */
int domino_head_param_count(const domino_head_config *cfg, int64_t *n);

/* Releases the handle (not the workspace or the weights).  NULL is a no-op. */
void domino_head_destroy(domino_head_t hd);

/* Message of the last failed call on this thread ("" if none). */
const char *domino_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DOMINO_HEAD_H */
