/*
 * flce.h - C ABI of libflce: chunked fused linear cross-entropy on gfx950.
 *
 * The operation (Liger Kernel pages: the ms-swift blog page, mechanism
 * paragraph, describes fused linear cross entropy as the last linear layer
 * merged with the cross-entropy loss; the project overview page, "Método de
 * API de Baixo Nível", calls it as loss_fn(weight, input, target) with
 * weight = nn.Linear(H, V).weight):
 *
 *     Z       = X W^T                                  [N, V], never stored whole
 *     loss    = (1 / N_valid) * sum_{i: y_i != ii} (logsumexp(Z_i) - Z_{i, y_i})
 *     G       = (softmax(Z) - onehot(y)) / N_valid     (0 on ignored rows)
 *     dX      = G W        dW = G^T X
 *
 * The work runs over consecutive chunks of tokens (overview page, "Computação
 * em Chunk"), so scratch memory is bounded by the chunk size, not by N x V.
 * Within a chunk the logits are rewritten in place into G (overview page,
 * "Operações In-Place").  The result is exact up to floating-point rounding
 * (overview page, "Implementação Técnica").
 *
 * Built on the same chunk pipeline: other reductions and per-token outputs
 * (flce_fwd_bwd_ex), cross-entropy on given logits (flce_ce_*), and the
 * fused-linear post-training losses of the overview page's list: ORPO, SimPO,
 * CPO, DPO (flce_orpo_*, flce_pair_*) and KTO (flce_kto_*).
 *
 * Conventions for every entry point:
 *   - All arrays are row-major and contiguous: X [N, H], W [V, H], dX [N, H],
 *     dW [V, H], labels [N].
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary host memory.  The caller owns every buffer; the
 *     library allocates no device memory.  The workspace is a caller-provided
 *     device buffer of at least flce_workspace_bytes(...) bytes, 256-byte
 *     aligned; its contents on entry do not matter.
 *   - stream is a hipStream_t (NULL = the default stream).  All device work is
 *     enqueued on it.  flce_fwd_bwd and flce_fwd synchronise the stream once,
 *     at the end, to return the loss and the label check.
 *   - Argument errors are detected on the host before any device work and
 *     return FLCE_EINVAL / FLCE_EUNSUPPORTED / FLCE_EWORKSPACE; outputs are
 *     then untouched.  Errors are never thrown across the ABI.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_EINVAL = 1,       /* bad argument: null pointer, negative size, unknown dtype, misalignment */
  FLCE_ELABEL = 2,       /* a label is neither ignore_index nor in [0, V); outputs unspecified */
  FLCE_EWORKSPACE = 3,   /* workspace_bytes < flce_workspace_bytes(...) */
  FLCE_EHIP = 4,         /* a HIP call failed; see flce_last_error() */
  FLCE_EUNSUPPORTED = 5  /* valid but unsupported shape: bf16 needs H % 8 == 0 and 16-byte aligned
                            X, W, dX; N < 2^31, H <= 2^20, V <= 8,000,000, chunks <= 2^23
                            tokens, and no launch of the call above 2^32 work-items */
} flce_status;

typedef enum {
  FLCE_F32 = 0,          /* X, W, dX in fp32; scratch in fp32 */
  FLCE_BF16 = 1          /* X, W, dX in bf16; fp32 accumulation; logits (less each token's partial
                            maximum, kept in fp32) and dlogits scratch in bf16 */
} flce_dtype;

/* How the per-token losses l_i = lse_i - z_{i,y_i} of valid tokens are reduced. */
typedef enum {
  FLCE_REDUCE_MEAN = 0,  /* loss = sum_i l_i / max(N_valid, 1) (flce_fwd_bwd, flce_fwd) */
  FLCE_REDUCE_SUM = 1,   /* loss = sum_i l_i */
  FLCE_REDUCE_NONE = 2   /* the output is the vector l (row_loss); loss = sum_i l_i */
} flce_reduction;

/*
 * Chunk planning.  The pages split memory-heavy work into chunks to cut peak
 * memory (project overview page, "Princípios Técnicos", Computação em
 * Chunk); these calls choose the chunk and report what it costs.
 *
 * The workspace of a call holds, for one chunk of C tokens: its logits, then
 * dlogits, in place ([C, V] bf16, or fp32 on the fp32 path), its X in the
 * GEMM operand layout and, for the backward, transposed in it too (bf16
 * path), the per-vocabulary-tile log-sum-exp
 * partials, per-token statistics and the split-K partial sums of dX; plus
 * one fp32 per-token loss for all N tokens.  Only that last array grows with
 * N; nothing grows with W beyond the chunk's logits (W is read in place).
 *
 * Budget used when a call plans its own chunk (chunk_tokens <= 0) and none is
 * given: the bytes of W in its dtype, but at least this floor.
 */
#define FLCE_DEFAULT_SCRATCH_FLOOR ((size_t)256 << 20)

/*
 * Bytes of workspace a call with these sizes and this chunk needs (the whole
 * workspace described above).  chunk_tokens <= 0 means "auto", as chosen by
 * flce_plan with the default budget; chunk_tokens > N is clamped to N, and any
 * chunk to at most 2^23 tokens.  Returns 0 for invalid sizes or dtype.  Host
 * only; no device call.
 */
size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_tokens);

/*
 * Choose the chunk and report the peak scratch of a call.
 *   chunk_tokens  in/out.  On entry the requested chunk: > 0 is used as
 *                 given (clamped to N and 2^23); <= 0 asks for the largest
 *                 power-of-two multiple of 256 tokens, at most N, whose whole
 *                 workspace fits scratch_budget_bytes.  On return the chunk a
 *                 call will use.
 *   scratch_budget_bytes  bound on the whole workspace;
 *                 0 = the default budget above.
 *   peak_scratch_bytes  out (may be NULL): the workspace the returned chunk
 *                 needs, which is the peak device scratch of a call.
 * Returns FLCE_OK; FLCE_EWORKSPACE when even the smallest chunk (256 tokens,
 * or N if fewer) does not fit the budget, or an explicit chunk exceeds an
 * explicit budget (*chunk_tokens and *peak_scratch_bytes still report that
 * chunk); FLCE_EUNSUPPORTED when a launch of the call would exceed 2^32
 * work-items; FLCE_EINVAL / FLCE_EUNSUPPORTED for invalid sizes, as the
 * calls below.  Host only; no device call.
 */
int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t *chunk_tokens,
              size_t scratch_budget_bytes, size_t *peak_scratch_bytes);

/*
 * Forward and backward in one call.
 *   X          device [N, H] (dtype)        read only
 *   W          device [V, H] (dtype)        read only
 *   labels     device [N] int64             read only; ignore_index marks ignored tokens
 *   loss       host   float                 mean loss over valid tokens (0 if none)
 *   dX         device [N, H] (dtype)        overwritten with dLoss/dX (rows of ignored tokens are 0)
 *   dW         device [V, H] fp32           overwritten with dLoss/dW (not accumulated into)
 *   row_loss   device [N] fp32 or NULL      per-token loss lse_i - z_{i,y_i} (0 if ignored)
 *   row_lse    device [N] fp32 or NULL      per-token log-sum-exp of the logits row
 *   workspace  device scratch, workspace_bytes long
 * N == 0 is allowed: loss = 0 and dW = 0.
 */
int flce_fwd_bwd(const void *X, const void *W, const int64_t *labels,
                 int64_t N, int64_t H, int64_t V, int dtype,
                 int64_t ignore_index, int64_t chunk_tokens,
                 float *loss, void *dX, float *dW,
                 float *row_loss, float *row_lse,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * flce_fwd_bwd with the workspace taken from a device array inside the
 * library, FLCE_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on,
 * held until the process ends.  The call allocates nothing.
 *   Arguments and results as for flce_fwd_bwd, without the workspace.
 *   chunk_tokens <= 0 plans the largest chunk whose workspace fits the array.
 *   A call whose workspace (flce_workspace_bytes with its chunk) exceeds the
 *   array returns FLCE_EWORKSPACE before any device work
 *   (flce_last_error() gives the sizes).
 *   The current device must be the stream's device.
 *   Every call on one GPU uses the same array: calls that overlap in time on
 *   one GPU race.  The first call on a GPU looks up the array's address there.
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
size_t flce_noalloc_scratch_bytes(void);
int flce_fwd_bwd_noalloc(const void *X, const void *W, const int64_t *labels,
                         int64_t N, int64_t H, int64_t V, int dtype,
                         int64_t ignore_index, int64_t chunk_tokens,
                         float *loss, void *dX, float *dW,
                         float *row_loss, float *row_lse, void *stream);

/*
 * Forward only: the loss (and optional per-token outputs) without gradients.
 * Arguments as for flce_fwd_bwd.  Needs no more workspace than flce_fwd_bwd.
 */
int flce_fwd(const void *X, const void *W, const int64_t *labels,
             int64_t N, int64_t H, int64_t V, int dtype,
             int64_t ignore_index, int64_t chunk_tokens,
             float *loss, float *row_loss, float *row_lse,
             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward and backward with a choice of reduction and extra per-token
 * outputs: the differentiated objective is L = sum_i w_i l_i over valid
 * tokens, with
 *   w_i = 1 / max(N_valid, 1)               reduction FLCE_REDUCE_MEAN
 *   w_i = 1                                 reduction FLCE_REDUCE_SUM
 *   w_i = grad_rows[i] (1 if grad_rows is NULL)   reduction FLCE_REDUCE_NONE
 * (for FLCE_REDUCE_NONE, grad_rows is the upstream gradient of the per-token
 * loss vector), so G_i = w_i (softmax(Z_i) - onehot(y_i)), dX = G W, dW = G^T X.
 * The per-token log-probabilities of the targets feed token-level losses
 * built on top of this one (project overview page, "Exemplo de Uso de Perda
 * de Pós-Treinamento").
 *   reduction      flce_reduction
 *   grad_rows      device [N] fp32 or NULL  only with FLCE_REDUCE_NONE (else FLCE_EINVAL)
 *   accumulate_dw  0: dW = dL/dW;  1: dW += dL/dW (dW holds valid fp32 values on entry)
 *   loss           host float               as flce_reduction says
 *   row_loss       device [N] fp32          per-token loss; required for FLCE_REDUCE_NONE (N > 0)
 *   row_lse        device [N] fp32 or NULL  per-token log-sum-exp
 *   logprob        device [N] fp32 or NULL  per-token z_{i,y_i} - lse_i (0 if ignored)
 * Other arguments and behaviour as for flce_fwd_bwd (with reduction MEAN,
 * grad_rows NULL, accumulate_dw 0 and logprob NULL it is flce_fwd_bwd).
 * N == 0: loss = 0; dW = 0, or unchanged when accumulating.
 */
int flce_fwd_bwd_ex(const void *X, const void *W, const int64_t *labels,
                    int64_t N, int64_t H, int64_t V, int dtype,
                    int64_t ignore_index, int64_t chunk_tokens,
                    int reduction, const float *grad_rows, int accumulate_dw,
                    float *loss, void *dX, float *dW,
                    float *row_loss, float *row_lse, float *logprob,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward only, with a choice of reduction and the per-token outputs of
 * flce_fwd_bwd_ex (row_loss is required for FLCE_REDUCE_NONE).
 */
int flce_fwd_ex(const void *X, const void *W, const int64_t *labels,
                int64_t N, int64_t H, int64_t V, int dtype,
                int64_t ignore_index, int64_t chunk_tokens, int reduction,
                float *loss, float *row_loss, float *row_lse, float *logprob,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Cross-entropy on given logits (no projection), the plain cross-entropy loss
 * the Liger Kernel pages list beside the fused one (project overview page,
 * "Modelos e Operações"); its gradient overwrites the logits (overview page,
 * "Princípios Técnicos", in-place operations):
 *     loss = reduce_i (lse(logits_i) - logits_{i,y_i})   over valid tokens
 *     logits_i := w_i (softmax(logits_i) - onehot(y_i))  (0 on ignored rows)
 * with reduce and w_i as for flce_fwd_bwd_ex.
 *   logits     device [N, V] (dtype)         flce_ce_fwd_bwd: read, then overwritten
 *                                            with dL/dlogits; flce_ce_fwd: read only
 *   labels     device [N] int64              read only
 *   reduction  flce_reduction; grad_rows as for flce_fwd_bwd_ex
 *   loss       host float
 *   row_loss, row_lse, logprob   device [N] fp32 or NULL (row_loss required for NONE)
 *   workspace  device, >= flce_ce_workspace_bytes(N) bytes, 256-byte aligned
 * logits must be aligned to its element size; 16-byte alignment with V a
 * multiple of 16 bytes' worth of elements takes the vector path.  On
 * FLCE_ELABEL the logits are already overwritten (unspecified).
 */
size_t flce_ce_workspace_bytes(int64_t N);
int flce_ce_fwd_bwd(void *logits, const int64_t *labels, int64_t N, int64_t V, int dtype,
                    int64_t ignore_index, int reduction, const float *grad_rows,
                    float *loss, float *row_loss, float *row_lse, float *logprob,
                    void *workspace, size_t workspace_bytes, void *stream);
int flce_ce_fwd(const void *logits, const int64_t *labels, int64_t N, int64_t V, int dtype,
                int64_t ignore_index, int reduction,
                float *loss, float *row_loss, float *row_lse, float *logprob,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Odds-ratio preference loss (ORPO) on the fused projection, one of the
 * fused-linear post-training losses of the Liger Kernel pages (project
 * overview page, "Kernels de Pós-Treinamento"; called as
 * orpo_loss(lm_head.weight, x, target) in "Exemplo de Uso de Perda de
 * Pós-Treinamento").  The pages give no formula; this is the published
 * definition (Hong, Lee and Thorne, 2024):
 *     a_s   = mean of log p(y_t) over the scored tokens of sequence s
 *     d_i   = log odds(a_chosen_i) - log odds(a_rejected_i),  log odds(a) = a - log(1 - e^a)
 *     loss  = NLL + beta * (1 / n_pairs) sum_i -log sigmoid(d_i)
 *     NLL   = mean of -log p(y_t) over the chosen sequences' scored tokens
 * with p = softmax(x_t W^T).  A pair with a sequence that has no scored token
 * adds nothing to the odds-ratio term.
 *   X          device [2 n_pairs T, H] (dtype)  2 n_pairs sequences of T rows: the
 *                                               n_pairs chosen ones, then the rejected
 *                                               ones; pair i = (sequence i, n_pairs + i)
 *   labels     device [2 n_pairs T] int64       ignore_index marks unscored tokens
 *   W          device [V, H] (dtype)
 *   beta       weight of the odds-ratio term
 *   chunk_pairs  pairs per chunk (a chunk holds both sequences of each of its
 *              pairs: 2 chunk_pairs T rows); <= 0: the largest count with at
 *              most 4096 rows (at least 1); at most n_pairs and 2^30 rows
 *   loss, nll  host float (nll may be NULL)
 *   dX         device [2 n_pairs T, H] (dtype), overwritten; dW device [V, H] fp32, overwritten
 *   chosen_logp, rejected_logp, log_odds_ratio   device [n_pairs] fp32 or NULL
 *   workspace  device, >= flce_orpo_workspace_bytes(...) bytes, 256-byte aligned
 * Same alignment rules and errors as flce_fwd_bwd; n_pairs, T >= 1.
 */
size_t flce_orpo_workspace_bytes(int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                                 int64_t chunk_pairs);
int flce_orpo_fwd_bwd(const void *X, const void *W, const int64_t *labels, int64_t n_pairs,
                      int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index, float beta,
                      int64_t chunk_pairs, float *loss, float *nll, void *dX, float *dW,
                      float *chosen_logp, float *rejected_logp, float *log_odds_ratio,
                      void *workspace, size_t workspace_bytes, void *stream);
int flce_orpo_fwd(const void *X, const void *W, const int64_t *labels, int64_t n_pairs, int64_t T,
                  int64_t H, int64_t V, int dtype, int64_t ignore_index, float beta,
                  int64_t chunk_pairs, float *loss, float *nll, float *chosen_logp,
                  float *rejected_logp, float *log_odds_ratio, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * The other pairwise preference losses of the same list (project overview
 * page, "Kernels de Pós-Treinamento"), each in its published form, on the
 * batch layout, chunking and outputs of flce_orpo_fwd_bwd.  With S = sum and
 * a = S / n = mean of log p(y_t) over a sequence's n scored tokens:
 *   FLCE_PAIR_ORPO   z = log odds(a_c) - log odds(a_r)            (lambda = beta)
 *   FLCE_PAIR_SIMPO  z = beta (a_c - a_r) - gamma                 (Meng, Xia and Chen, 2024)
 *   FLCE_PAIR_CPO    z = beta (S_c - S_r)                         (Xu et al., 2024)
 *   FLCE_PAIR_DPO    z = beta ((S_c - R_c) - (S_r - R_r))         (Rafailov et al., 2023)
 *   loss = alpha NLL + lambda (1 / n_pairs) sum_i -log sigmoid(z_i),  lambda = 1 unless ORPO
 * R_c, R_r: device [n_pairs] fp32, the reference model's sequence log-probability sums
 * (required for DPO, ignored otherwise).  chosen_logp / rejected_logp receive the
 * sequence log-probability the loss uses (a for ORPO and SimPO, S for CPO and DPO),
 * pair_logit receives z.  An unknown kind is FLCE_EINVAL.
 */
typedef enum {
  FLCE_PAIR_ORPO = 0,
  FLCE_PAIR_SIMPO = 1,
  FLCE_PAIR_CPO = 2,
  FLCE_PAIR_DPO = 3
} flce_pair_loss;
size_t flce_pair_workspace_bytes(int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                                 int64_t chunk_pairs);
int flce_pair_fwd_bwd(int kind, const void *X, const void *W, const int64_t *labels,
                      int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                      int64_t ignore_index, float beta, float gamma, float alpha,
                      const float *ref_chosen_logp, const float *ref_rejected_logp,
                      int64_t chunk_pairs, float *loss, float *nll, void *dX, float *dW,
                      float *chosen_logp, float *rejected_logp, float *pair_logit,
                      void *workspace, size_t workspace_bytes, void *stream);
int flce_pair_fwd(int kind, const void *X, const void *W, const int64_t *labels, int64_t n_pairs,
                  int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index, float beta,
                  float gamma, float alpha, const float *ref_chosen_logp,
                  const float *ref_rejected_logp, int64_t chunk_pairs, float *loss, float *nll,
                  float *chosen_logp, float *rejected_logp, float *pair_logit, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * The unpaired loss of the same list: KTO (Ethayarajh et al., 2024).  The rows
 * of X are n_seq sequences of T tokens (no pairing); with S the sum of
 * log p(y_t) over a sequence's scored tokens, R its reference value and
 * r = S - R,
 *     desirable:    l = lambda_d (1 - sigmoid(beta (r - z0)))
 *     undesirable:  l = lambda_u (1 - sigmoid(beta (z0 - r)))
 *     loss = mean over sequences of l
 * z0 is the reference point (a host value; no gradient flows through it).
 *   desirable  device [n_seq] int32, nonzero marks a desirable sequence
 *   ref_logp   device [n_seq] fp32, R (required)
 *   chunk_seqs sequences per chunk; <= 0: the largest count with at most 4096 rows
 *              (at least 1); at most n_seq and 2^30 rows
 *   logp, reward  device [n_seq] fp32 or NULL: S and r
 * Other arguments, alignment and errors as for flce_orpo_fwd_bwd.
 */
size_t flce_kto_workspace_bytes(int64_t n_seq, int64_t T, int64_t H, int64_t V, int dtype,
                                int64_t chunk_seqs);
int flce_kto_fwd_bwd(const void *X, const void *W, const int64_t *labels, int64_t n_seq,
                     int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                     const int32_t *desirable, const float *ref_logp, float beta, float z0,
                     float lambda_d, float lambda_u, int64_t chunk_seqs, float *loss, void *dX,
                     float *dW, float *logp, float *reward, void *workspace,
                     size_t workspace_bytes, void *stream);
int flce_kto_fwd(const void *X, const void *W, const int64_t *labels, int64_t n_seq, int64_t T,
                 int64_t H, int64_t V, int dtype, int64_t ignore_index, const int32_t *desirable,
                 const float *ref_logp, float beta, float z0, float lambda_d, float lambda_u,
                 int64_t chunk_seqs, float *loss, float *logp, float *reward, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * KTO's reference point z0, estimated from a batch the way its published
 * definition does: the rows of X are n_seq completions, each scored under a
 * prompt that is not its own (mismatched pairs), ref_logp their reference
 * sums R; with S the policy's sum of log p(y_t) over a sequence's scored
 * tokens,
 *     z0 = max(0, (1 / n_seq) sum_s (S_s - R_s))
 * computed on the device (forward only, fp64 mean), with no gradient.  The
 * result is the host float *z0 that flce_kto_fwd_bwd takes.
 *   X, W, labels, n_seq, T, H, V, dtype, ignore_index, chunk_seqs, workspace
 *              as for flce_kto_fwd_bwd (workspace >= flce_kto_workspace_bytes(...))
 *   ref_logp   device [n_seq] fp32, R (required)
 *   z0         host float, out
 *   logp, reward  device [n_seq] fp32 or NULL: S and S - R
 * Same alignment rules and errors as flce_kto_fwd_bwd.
 */
int flce_kto_reference_point(const void *X, const void *W, const int64_t *labels, int64_t n_seq,
                             int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                             const float *ref_logp, int64_t chunk_seqs, float *z0, float *logp,
                             float *reward, void *workspace, size_t workspace_bytes, void *stream);

/*
 * buf[i] *= *scale for i < n, in place, on the stream (no sync).  buf is a
 * device array of dtype (FLCE_F32 or FLCE_BF16); scale is a device fp32
 * scalar.  Used to apply an upstream gradient d(out)/d(loss) != 1 to dX, dW.
 */
int flce_scale_inplace(void *buf, int64_t n, int dtype, const float *scale, void *stream);

/*
 * Per-kernel timing.  While enabled (process-wide), every kernel launch of
 * the entry points above whose class is selected (flce_profile_select; all
 * classes by default) is bracketed by a pair of HIP events on the call's
 * stream.  flce_profile_read waits for the recorded events, writes the
 * summed milliseconds and the launch count of each kernel class k < n
 * (FLCE_K_*) into ms[k] and launches[k] (either may be NULL), and clears the
 * records.  Both return FLCE_OK or FLCE_EHIP.
 */
enum {
  FLCE_K_LABELS = 0,      /* label check and N_valid */
  FLCE_K_FWD_TILE = 1,    /* forward GEMM tile + log-sum-exp epilogue */
  FLCE_K_LSE_COMBINE = 2, /* combine of the per-tile partials */
  FLCE_K_DLOGITS = 3,     /* in-place rewrite of logits into dlogits */
  FLCE_K_DX_GEMM = 4,     /* dX split-K GEMM */
  FLCE_K_DX_REDUCE = 5,   /* dX split-K reduction */
  FLCE_K_DW_GEMM = 6,     /* dW GEMM */
  FLCE_K_FINAL = 7,       /* final mean loss, fills */
  FLCE_K_PACK = 8,        /* per-chunk packing of X (and X transposed) into the GEMM operand layout */
  FLCE_K_CE_ROWS = 9,     /* cross-entropy on given logits, one workgroup per row */
  FLCE_K_PAIRS = 10,      /* preference losses: label pass, per-pair step, final loss */
  FLCE_K_PAIR_ROWS = 11,  /* preference losses: gathering a chunk's rows, scattering dX */
  FLCE_K_COUNT = 12
};
int flce_profile_enable(int enable);
int flce_profile_read(double *ms, int64_t *launches, int n);
/*
 * Which kernel classes get events while timing is enabled: bit k of
 * class_mask for class k (process-wide; all classes until first called).
 * Lets a caller time a run with events on a few launches only, since every
 * event pair costs the stream a little.  Host only; returns FLCE_OK.
 */
int flce_profile_select(uint32_t class_mask);

/* Static name of a kernel class (FLCE_K_*), "" if out of range. */
const char *flce_kernel_name(int k);

/* Static text for a status code. */
const char *flce_status_string(int status);

/* Text of the last FLCE_EHIP error raised on the calling thread ("" if none). */
const char *flce_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
