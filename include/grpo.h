/*
 * grpo.h — C ABI of libgrpo, the memory-efficient linear GRPO loss on MI355X (gfx950).
 *
 * The loss, as the pages define it [Long-context GRPO (note.com), §2-§4; Train your own
 * R1 reasoning model with Unsloth, §3]:
 *
 *   For G sampled completions of one prompt, the policy's and the reference model's final
 *   hidden states X_q, X_p [S*L, H] are projected through one lm_head W [V, H] to
 *   per-token log-probs of the sampled tokens, q and ref, by a logsumexp over the
 *   vocabulary.  The (G, L, V) logits are never stored: the vocabulary is swept in
 *   chunks with an online max / sum-of-exponentials.  Per loss token t of sequence s
 *
 *       KL_t = exp(ref_t - q_t) - (ref_t - q_t) - 1          (reverse-KL estimator)
 *       l_t  = beta * KL_t - A_s                              (value of -(ratio*A - beta*KL),
 *                                                              ratio = exp(q - sg(q)) = 1)
 *       loss = sum_t m_t * l_t / max(1, sum_t m_t)            (mean over completion tokens)
 *
 *   The gradient flows through q only: dloss/dq_t = m_t * (-A_s - beta*(exp(ref_t-q_t)-1))
 *   / N_tok, and dq_t/dz_t = onehot(y_t) - softmax(z_t) with z_t = W x_q[t].  The backward
 *   recomputes the same vocabulary chunks instead of storing softmax.
 *
 *   Advantages are group-relative: A_s = (r_s - mean_g r) / (std_g r + eps), where r_s is
 *   the sum of the K reward-function scores of completion s and std is the unbiased
 *   (G - 1) standard deviation.
 *
 * Conventions common to every entry point
 *   - Every pointer argument except scalars is DEVICE memory, owned by the caller.  The
 *     library never allocates, never synchronises the host with the device, never prints
 *     and never aborts.  All work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) in order, and may still be running when the call returns.
 *   - Matrices are row-major and dense: X_q, X_p, dX_q are [S*L, H] with row t = position
 *     t % L of sequence t / L; W is [V, H].  H must be a positive multiple of 8 (16-byte
 *     rows of 16-bit data); 16-bit inputs with H a multiple of 256 run on the MFMA
 *     kernels, everything else on fp32-accumulating FMA kernels.  V is arbitrary (ragged
 *     vocabulary tails are handled).  S * L must fit in int32.
 *   - `targets[t]` is the token that row t's hidden state predicts (the caller has already
 *     shifted ids by one position).  Rows with mask 0 are never read and their outputs are 0;
 *     a NaN in a masked-out row therefore sets no flag.
 *   - Invalid arguments return a negative grpo_status before anything is enqueued.  Launch
 *     failures return GRPO_ERR_HIP.  Data-dependent problems (non-finite values, a target
 *     outside [0, V) on a loss row) are reported through device-side flag words.
 *   - Calls that share a workspace must not overlap in time (same stream, or synchronised).
 *   - A workspace's contents on entry do not matter: every call writes what it reads, and
 *     grpo_loss_bwd takes nothing from the workspace of the forward before it.
 */
#ifndef GRPO_H_
#define GRPO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* grpo_stream_t; /* hipStream_t */

typedef enum grpo_dtype {
  GRPO_F32 = 0,  /* fp32 operands, fp32 FMA products (parity workloads) */
  GRPO_BF16 = 1, /* bfloat16 operands, MFMA with fp32 accumulation      */
  GRPO_F16 = 2   /* IEEE half operands, MFMA with fp32 accumulation     */
} grpo_dtype;

typedef enum grpo_status {
  GRPO_OK = 0,
  GRPO_ERR_NULL = -1,      /* a required pointer is NULL                                  */
  GRPO_ERR_SHAPE = -2,     /* a size is out of range (G < 2, H not a multiple of 8, ...)  */
  GRPO_ERR_DTYPE = -3,     /* unknown grpo_dtype                                          */
  GRPO_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned                            */
  GRPO_ERR_WORKSPACE = -5, /* workspace smaller than grpo_workspace_bytes()               */
  GRPO_ERR_HIP = -6,       /* the HIP runtime reported an error when enqueuing           */
  GRPO_ERR_DEVICE = -7,    /* the current device is not a gfx950 GPU                      */
  GRPO_ERR_OPTIONS = -8,   /* a grpo_options field is out of range, or not supported for  */
                           /* these inputs (fp8_logits with fp32 data)                     */
  GRPO_ERR_SCRATCH = -9,   /* grpo_loss_fwd_noalloc: the forward of these sizes needs more */
                           /* than GRPO_NOALLOC_SCRATCH_BYTES                              */
  GRPO_ERR_HOST = -10      /* a host buffer of the gradient offload is not pinned host     */
                           /* memory (hipHostMalloc) over its whole extent                 */
} grpo_status;

/* Loss variants: the four experiments of [Long-context GRPO, §4] and two readings the
 * pages leave open.  A NULL options pointer selects the defaults (first value of each). */
typedef enum grpo_kl_estimator {
  GRPO_KL_REVERSE = 0,    /* exp(ref - q) - (ref - q) - 1: reverse KL(Q||P), no Q factor    */
  GRPO_KL_FORWARD = 1,    /* exp(q - ref) - (q - ref) - 1: the same estimator, roles swapped */
  GRPO_KL_REVERSE_Q = 2   /* exp(q) * (exp(ref - q) - (ref - q) - 1): the reverse estimator
                             with the extra Q(y) factor the pages discuss (their formula was
                             lost; this is the reading implemented)                          */
} grpo_kl_estimator;

typedef enum grpo_normalization {
  GRPO_NORM_TOKENS = 0,   /* loss = sum_t m_t l_t / N_tok (mean over all completion tokens) */
  GRPO_NORM_SEQUENCES = 1 /* loss = mean over sequences with tokens of their token means     */
} grpo_normalization;

/* Kernels whose launches grpo_options.trace_kernel can bracket with events. */
typedef enum grpo_trace_kernel {
  GRPO_TRACE_NONE = 0,
  GRPO_TRACE_FWD_ALL = 1,   /* the forward GEMM over all loss rows: both sides (grpo_loss_fwd)
                               or the reference side (grpo_loss_fwd_bwd)                     */
  GRPO_TRACE_FWD_CHUNK = 2, /* single pass: one chunk's policy forward that keeps its terms  */
  GRPO_TRACE_RECOMPUTE = 3, /* two-pass backward: one chunk's onehot - softmax               */
  GRPO_TRACE_DX = 4,        /* one chunk's dX GEMM                                            */
  GRPO_TRACE_DW = 5         /* one chunk's dW GEMM                                            */
} grpo_trace_kernel;

typedef struct grpo_options {
  int kl_estimator;       /* grpo_kl_estimator                                             */
  int detach_ratio;       /* 1: advantage times exp(q - sg(q)) (value 1, gradient A dq);
                             0: exp(q - q), whose gradient vanishes (the no-detach experiment) */
  int normalization;      /* grpo_normalization                                            */
  float temperature;      /* logits are divided by it before the log-softmax; in [1e-3, 1e3] */
  int fp8_logits;         /* 1: both sides' logits from per-row e4m3 copies of X and W
                             (scale amax / 448 per row, see grpo_quantize_e4m3); gradients
                             still use the original X and W.  16-bit inputs with H a
                             multiple of 256 only.  Needs grpo_workspace_bytes_opts.      */
  int chunk_rows;         /* loss rows per backward chunk: 0 = 4096; else a multiple of 256
                             in [256, 65536].  The workspace holds one chunk of rows x V
                             16-bit entries, so this trades workspace for speed (fewer,
                             larger GEMM launches); results do not depend on it beyond
                             fp32 summation order.  Needs grpo_workspace_bytes_opts.      */
  int vocab_piece;        /* vocabulary entries per piece of a chunk's softmax terms when the
                             backward is split over the vocabulary (16-bit inputs on the
                             MFMA kernels, except grpo_loss_fwd_bwd with dW): 0 = about
                             32768 (pieces balanced over V); else a multiple of 256.  The
                             workspace holds one chunk of rows x one piece, plus fp32 dX
                             sums of one chunk.  Needs grpo_workspace_bytes_opts.          */
  /* Timing of one kernel as launched inside a call (16-bit MFMA path; the fp32 kernels are
   * not bracketed).  trace_events: hipEvent_t[2 * trace_capacity], created by the caller
   * with timing enabled; the library records events 2i and 2i + 1 on the call's stream
   * just before and just after the i-th launch of the kernel named by trace_kernel (the
   * gated fallback launches excepted), up to trace_capacity launches, and stores the
   * number of such launches in *trace_count (host memory, written before the call returns;
   * may be NULL).  trace_kernel 0 records nothing.                                        */
  int trace_kernel;       /* grpo_trace_kernel                                             */
  int trace_capacity;
  void* const* trace_events;
  int* trace_count;
  /* Gradient offload of grpo_loss_fwd_bwd to host memory: what a training step holds
   * between its forward and its backward goes to system RAM asynchronously, at a small
   * cost in step time [Long-context GRPO (note.com), §2, the offloaded activations].
   * dx_host: NULL, or pinned host memory (hipHostMalloc) of S*L rows x H in `dtype`, 16-byte
   * aligned.  When set, dXq must be NULL and no device dX is written: each chunk's dX rows
   * go to one of two staging slots in the workspace and are copied from there to dx_host on
   * copy_stream while the next chunks compute.  Row r of dx_host then holds the gradient of
   * the r-th loss row (mask = 1 rows in order); the rows past the loss-row count are
   * undefined.  dw_host: NULL, or pinned host memory of V x H fp32, which receives dW (still
   * accumulated in the dW given to the call) after the last chunk.  copy_stream: required
   * when either is set, not the call's stream; a stream of the same device, created with
   * the default priority.  The copies run on the SDMA engines, beside the kernels.  Before
   * the call returns, `stream` is made to wait for them, so that work enqueued on it
   * afterwards (grpo_grad_restore, an event) finds the host buffers complete; a host
   * buffer that is not pinned memory over its extent is rejected with GRPO_ERR_HOST.
   * grpo_grad_restore brings the gradients back.  The workspace grows by two chunks of
   * rows x H (grpo_workspace_bytes_opts).                                                  */
  void* dx_host;
  void* dw_host;
  grpo_stream_t copy_stream;
} grpo_options;

/* Bits of the forward's status word. */
#define GRPO_FLAG_NONFINITE 1   /* loss, a log-prob, KL or g of a loss row is inf/NaN */
#define GRPO_FLAG_BAD_TARGET 2  /* a loss row's target lies outside [0, V)             */

/* Human-readable name of a grpo_status value (static storage). */
const char* grpo_status_string(int status);

/* Bytes of device workspace that grpo_loss_fwd and grpo_loss_bwd need for these sizes
 * (S = sequences, L = positions per sequence) with the default options.  The same
 * workspace can serve both calls.  It grows with one chunk of rows times V (and with the
 * rows S*L through 16-byte per-row partials), never with S*L*V.  Returns 0 if the sizes
 * are invalid. */
size_t grpo_workspace_bytes(int64_t S, int64_t L, int64_t H, int64_t V, grpo_dtype dtype,
                            int need_dW);

/* The same for a loss variant (opts may be NULL): fp8_logits adds the e4m3 copies of W and
 * of the loss rows of X_q and X_p (N H + V H bytes and their scales); chunk_rows sets the
 * chunk.  Returns 0 if the sizes or the options are invalid. */
size_t grpo_workspace_bytes_opts(int64_t S, int64_t L, int64_t H, int64_t V, grpo_dtype dtype,
                                 int need_dW, const grpo_options* opts);

/* Per-row fp8 e4m3 ("fn": maximum 448, no infinities) quantisation of a [rows, H] matrix:
 * amax = max |x| of the row, scales[r] = amax / 448 and dst[r][h] = e4m3(x * (448 / amax)),
 * with correctly rounded fp32 division and product and round-to-nearest-even onto the
 * e4m3 grid (a row of zeros gets scale 1; a row holding inf or NaN gets scale NaN).  This
 * is the quantisation of the fp8_logits option, exported for callers that keep fp8
 * weights.  dst: uint8 [rows, H]; scales: fp32 [rows]; H a multiple of 4. */
int grpo_quantize_e4m3(const void* src, grpo_dtype dtype, int64_t rows, int64_t H,
                       uint8_t* dst, float* scales, grpo_stream_t stream);

/* Group-relative advantages [Train your own R1 reasoning model with Unsloth, §3;
 * Long-context GRPO, §4].
 *   rewards  fp32 [B, G, K]: score of completion g of prompt b under reward function k.
 *   adv      fp32 [B*G] out: A = (r - mean) / (std + eps), r summed over k first.
 *   unbiased 1: std divides by G - 1 (needs G >= 2); 0: divides by G.
 * Operations run in one fixed fp32 order (k ascending, then g ascending sums, no fused
 * multiply-add, correctly rounded division and square root), so results are
 * reproducible bit for bit. */
int grpo_advantages(const float* rewards, int64_t B, int64_t G, int64_t K, float eps,
                    int unbiased, float* adv, grpo_stream_t stream);

/* Defaults: reverse estimator, detached ratio, token mean, temperature 1, 16-bit logits,
 * chunks of 4096 rows, no tracing. */
void grpo_default_options(grpo_options* opts);

/* Forward: loss and per-token terms, without materialising logits
 * [Long-context GRPO, §2 (memory figures), §3 (the linear algorithm), §4 (KL, ratio,
 * logsumexp)].
 *   Xq, Xp   [S*L, H] in `dtype`: policy and reference final hidden states.
 *   W        [V, H] in `dtype`: the lm_head shared by policy and reference.
 *   targets  int64 [S*L]; mask uint8 [S*L] (1 = completion token counted in the loss);
 *   adv      fp32 [S]: one advantage per sequence (see grpo_advantages).
 *   loss     fp32 [1] out.
 *   saved    fp32 [S*L, 4] out: (lse_q, q, ref, dloss/dq) per row; the backward reads it.
 *   logp_out, ref_logp_out, kl_out: fp32 [S*L] out, each may be NULL.
 *   status   int32 [1] out: GRPO_FLAG_* bits of this call (overwritten, not accumulated).
 *   opts     loss variant, or NULL for the defaults; the backward must get the same one.
 *   workspace, workspace_bytes: at least grpo_workspace_bytes(..., need_dW = 0).
 * Xq, Xp, W, saved, workspace must be 16-byte aligned. */
int grpo_loss_fwd(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                  const int64_t* targets, const uint8_t* mask, const float* adv, int64_t S,
                  int64_t L, int64_t H, int64_t V, float beta, float* loss, float* saved,
                  float* logp_out, float* ref_logp_out, float* kl_out, int32_t* status,
                  const grpo_options* opts, void* workspace, size_t workspace_bytes,
                  grpo_stream_t stream);

/* Bytes of the fixed device array behind grpo_loss_fwd_noalloc (one per GPU). */
#define GRPO_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* grpo_loss_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and error behaviour as grpo_loss_fwd (bit for bit), without the workspace: the library
 * keeps the forward's working buffers in a fixed array of GRPO_NOALLOC_SCRATCH_BYTES in
 * device memory, one copy per GPU it runs on, held until the process ends.  The call
 * allocates nothing (the array's address is looked up once per device, on the first
 * call there).  Sizes whose forward needs more than the array holds return
 * GRPO_ERR_SCRATCH before anything is enqueued (with 16-bit logits the forward of every
 * documented workload fits except the 8 x 20480 long-context one; fp8_logits adds the
 * e4m3 copies of W and of the loss rows).  Every call on one GPU shares that array: calls that
 * overlap in time on one GPU (different streams, or threads) race and must not be made;
 * calls ordered on one stream are safe, and each call rewrites every part of the array it
 * reads. */
int grpo_loss_fwd_noalloc(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                          const int64_t* targets, const uint8_t* mask, const float* adv,
                          int64_t S, int64_t L, int64_t H, int64_t V, float beta, float* loss,
                          float* saved, float* logp_out, float* ref_logp_out, float* kl_out,
                          int32_t* status, const grpo_options* opts, grpo_stream_t stream);

/* Backward: dloss/dXq (and dloss/dW) by recomputing the vocabulary chunks.
 *   Xq, W, targets, mask, saved: as given to / produced by grpo_loss_fwd.
 *   grad_loss  fp32 [1] device, or NULL for 1.0: the upstream gradient of the loss.
 *   loss_scale the factor the caller scaled the loss by (1.0 without loss scaling).  The
 *              outputs are multiplied by grad_loss / loss_scale, so an fp16 caller that
 *              back-propagates S * loss passes S twice and gets unscaled gradients.  The
 *              per-token factors stay in fp32; 16-bit GEMM operands only ever hold
 *              onehot - softmax, which lies in [-1, 1], so loss scaling cannot overflow
 *              them (the mixed-precision hazard of [Long-context GRPO, §3]).
 *   dXq        [S*L, H] in `dtype`, out (masked rows are written as 0).
 *   dW         fp32 [V, H] out, or NULL to skip; accumulate_dW = 1 adds into it.
 *   found_inf  int32 [1] device: set to 1 if any element of dXq or dW is inf/NaN; never
 *              cleared by the library.
 *   opts       the options given to the forward (only the temperature is read here: the
 *              variant's dloss/dq is already in `saved`).
 *   workspace  at least grpo_workspace_bytes(..., need_dW = (dW != NULL)). */
int grpo_loss_bwd(const void* Xq, const void* W, grpo_dtype dtype, const int64_t* targets,
                  const uint8_t* mask, const float* saved, int64_t S, int64_t L, int64_t H,
                  int64_t V, const float* grad_loss, float loss_scale, void* dXq, float* dW,
                  int accumulate_dW, int32_t* found_inf, const grpo_options* opts,
                  void* workspace, size_t workspace_bytes, grpo_stream_t stream);

/* Forward and backward in one call: the loss and per-token terms of grpo_loss_fwd and the
 * gradients of grpo_loss_bwd, with the policy logits of each row computed once instead of
 * twice.  The reference side runs over all rows first; then, per chunk of rows, the policy
 * forward keeps its softmax terms in the workspace, taken against the row's reference-side
 * log-sum-exp, the chunk's loss terms are merged (which also rewrites each row's target
 * entry, so that the row is -(onehot - softmax) / f for a per-row f), and dX (and dW)
 * follow from the kept rows scaled by -f.  A chunk holding a row whose two log-sum-exps
 * lie more than 60 (in log2 units) apart is redone with terms taken against running
 * maxima, turned into onehot - softmax in place (for fp16, a row outside [-4, 14] does so:
 * the kept terms must fit fp16).  This is the chunked algorithm of
 * [Long-context GRPO, §3] with the
 * backward's recomputation of the chunk's logits replaced by the forward's own; memory
 * stays one chunk of rows times V.
 *   Arguments: those of grpo_loss_fwd, then grad_loss / loss_scale, dXq, dW,
 *   accumulate_dW and found_inf as in grpo_loss_bwd.  The upstream gradient must be known
 *   when the call is enqueued (grad_loss is read on the device; NULL means 1).  An
 *   autograd caller passes NULL and 1, keeps dXq (and dW), and applies its upstream
 *   gradient later with grpo_scale_grad.
 *   workspace: at least grpo_workspace_bytes(..., need_dW = (dW != NULL)).
 *   dXq may be NULL when opts->dx_host is set (the gradient offload, see grpo_options).
 * Results equal grpo_loss_fwd followed by grpo_loss_bwd up to rounding: the kept softmax
 * terms are rounded to the storage type once more than the recomputed ones.  fp32, and H
 * not a multiple of 256, run the two passes back to back inside this call. */
int grpo_loss_fwd_bwd(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                      const int64_t* targets, const uint8_t* mask, const float* adv, int64_t S,
                      int64_t L, int64_t H, int64_t V, float beta, const float* grad_loss,
                      float loss_scale, float* loss, float* saved, float* logp_out,
                      float* ref_logp_out, float* kl_out, int32_t* status, void* dXq, float* dW,
                      int accumulate_dW, int32_t* found_inf, const grpo_options* opts,
                      void* workspace, size_t workspace_bytes, grpo_stream_t stream);

/* Multiplies gradients in place by grad_loss / loss_scale (grad_loss: fp32 [1] on the
 * device; nothing is done when the factor is exactly 1): dXq [rows, H] in `dtype` and,
 * if dW is not NULL, dW fp32 [V, H].  found_inf is set to 1 on any non-finite result.
 * For the upstream gradient of a grpo_loss_fwd_bwd call made with grad_loss = 1.
 * H must be a multiple of 8; dXq and dW 16-byte aligned. */
int grpo_scale_grad(void* dXq, grpo_dtype dtype, int64_t rows, int64_t H, float* dW, int64_t V,
                    const float* grad_loss, float loss_scale, int32_t* found_inf,
                    grpo_stream_t stream);

/* Workspace of grpo_grad_restore: the loss-row list of S*L rows (0 for invalid sizes). */
size_t grpo_restore_workspace_bytes(int64_t S, int64_t L);

/* The way back of the gradient offload (grpo_options.dx_host / dw_host of
 * grpo_loss_fwd_bwd), with the upstream gradient applied as grpo_scale_grad applies it:
 *   dXq[t] = dx_host[k] * grad_loss / loss_scale for the k-th loss row t (mask[t] = 1),
 *            0 for the other rows;
 *   dW     = dw_host * grad_loss / loss_scale;
 * the product is skipped when the factor is exactly 1, so the results equal those of a
 * device-held gradient scaled by grpo_scale_grad, bit for bit.  The kernels read the pinned
 * host buffers directly over PCIe (no staging copy: in a backward there is no computation
 * of this op to overlap it with), enqueued on `stream` after the work already there.
 *   dx_host, dXq: both set or both NULL (dtype, S*L rows x H); dw_host, dW: both set or
 *   both NULL (fp32 V x H); at least one pair.  Host buffers must be pinned host memory
 *   over their whole extent (else GRPO_ERR_HOST, before anything is enqueued) and stay
 *   allocated until the kernels have run.
 *   mask      the forward's mask (loss rows are found again from it); needed with dx_host.
 *   grad_loss fp32 [1] device, or NULL for 1.0.
 *   found_inf int32 [1] device, set to 1 on a non-finite product (never cleared).
 *   workspace at least grpo_restore_workspace_bytes(S, L) (needed with dx_host).
 * dXq, dW and the host buffers 16-byte aligned; H a multiple of 8. */
int grpo_grad_restore(const void* dx_host, const float* dw_host, grpo_dtype dtype,
                      const uint8_t* mask, int64_t S, int64_t L, int64_t H, int64_t V,
                      const float* grad_loss, float loss_scale, void* dXq, float* dW,
                      int32_t* found_inf, void* workspace, size_t workspace_bytes,
                      grpo_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_H_ */
