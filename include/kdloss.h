/*
 * kdloss — fused, chunked sparse-KL distillation loss head for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The operation (Hugging Face blog "Making Knowledge Distillation Cheap Enough
 * to Run at Scale", section "Two systems changes"; arXiv 2608.03796 abstract;
 * aib.vote summary, paragraph comparing Dense, Forward-chunked and Fused
 * chunked KL): the student's output projection (logits z = H W^T over the
 * whole vocabulary) is fused with a full-vocabulary log-softmax and a KL
 * divergence against the teacher's cached top-K entries (the offline top-K
 * cache of that same section).  Rows are processed one chunk at a time; the
 * n x V logit matrix is never stored, and the backward call recomputes each
 * chunk's logits (the "fused chunked" variant), so device memory grows
 * linearly with n.
 *
 * Definition computed, per row t with teacher ids i_{t,k}, values a_{t,k}:
 *   log q_{t,v} = z_{t,v} - LSE_v(z_t)                 (full vocabulary)
 *   l_{t,k} = a_{t,k} - LSE_k(a_t),  p_{t,k} = exp(l)  (teacher renormalised over K)
 *   KL_t    = sum_k p_{t,k} (l_{t,k} - log q_{t,i_{t,k}})
 *   loss    = sum_{t: mask_t != 0} KL_t / N_valid       (0 if N_valid == 0)
 * and its gradient (the closed form the blog refers to in its closing
 * paragraph):  G_{t,v} = grad_loss * [mask_t] / N_valid * (S_t q_{t,v} -
 * sum_k p_{t,k} [i_{t,k} = v]),  S_t = sum_k p_{t,k};  dH = G W,  dW += G^T H.
 * No tail bucket: the teacher's mass lives only on its K ids.  At temperature
 * 1 this is the method as the blog describes it; a temperature and padding
 * entries are extensions, documented before the forward call.
 *
 * Layouts (all row-major, contiguous):
 *   H        [n, d]  dtype (bf16 or fp32)        student hidden states
 *   W        [V, d]  dtype                       output-projection weight
 *   topk_idx [n, K]  int32 < V                   teacher ids (< 0: padding; duplicates summed)
 *   topk_logp[n, K]  fp32                        teacher log-values (any per-row offset;
 *                                                -inf = zero probability)
 *   mask     [n]     uint8, NULL = all ones      0 removes the row entirely (its ids
 *                                                and values are never read)
 * All device pointers are allocated and owned by the caller; H, W, dH and dW
 * must be 16-byte aligned and d must be a multiple of 8 (bf16) or 4 (fp32).
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream)
 * and never synchronise the host, except when validation is switched on.
 * No C++ exception crosses this interface.  NaN / Inf in inputs propagate to
 * the outputs and are not reported as errors.
 */
#ifndef KDLOSS_H
#define KDLOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of H, W and dH (H and W share one). */
enum { KD_BF16 = 0, KD_F32 = 1 };

/* Status codes returned by every call. */
enum {
  KD_OK = 0,
  KD_E_INVAL = -1,     /* null pointer, size <= 0, K > V, misalignment, bad dtype or chunk */
  KD_E_WORKSPACE = -2, /* workspace too small (the message gives the bytes needed) or no plan fits */
  KD_E_HIP = -3,       /* a HIP runtime call or kernel launch failed */
  KD_E_RANGE = -4      /* a teacher id >= V on an unmasked row (validation mode only);
                          kd_teacher_topk: a row's candidate list overflowed */
};

/* Result of the chunk and workspace planner. */
typedef struct kd_plan {
  int64_t chunk;               /* rows per chunk (the last chunk may be shorter) */
  int64_t n_chunks;
  int64_t vocab_tiles;         /* 256-wide vocabulary tiles of the fused GEMMs */
  int64_t dh_splits;           /* split-K factor of the dH = G W contraction */
  size_t fwd_workspace_bytes;  /* needed by kd_fused_chunked_kl_fwd */
  size_t bwd_workspace_bytes;  /* needed by kd_fused_chunked_kl_bwd */
  size_t workspace_bytes;      /* max of the two: one buffer can serve both calls */
} kd_plan_t;

/*
 * Chooses the chunk size and reports the workspace each call needs.  The
 * chunk bounds the only per-chunk buffers (the logit-gradient slices of
 * chunk x V entries: G, and for fp32 also G^T); everything else is linear in n.
 * chunk > 0 is honoured as given (it must be a multiple of 64 unless it is
 * >= n).  chunk <= 0 lets the planner pick the largest multiple of 256 that is
 * <= 8192, <= max(256, n/2 rounded up to 256) and whose workspace fits in
 * min(hbm_budget, 24 GiB).  hbm_budget == 0 means: half of the device's free
 * memory (hipMemGetInfo on the current device); otherwise no device call is
 * made.  The same (dtype, n, d, V, K, chunk) always yields the same plan for
 * the same budget.
 */
int kd_plan_query(int dtype, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                  size_t hbm_budget, kd_plan_t* out);

/*
 * Teacher entries and temperature (both calls):
 *   topk_idx  [n, K] int32: vocabulary ids; an id < 0 marks a padding entry
 *             (rows with fewer than K cached entries): it has probability 0
 *             and is excluded from the renormalisation, whatever its log-value;
 *             an unmasked row needs at least one id >= 0 (an all-padding row
 *             has no teacher distribution: its results are NaN, so mask it)
 *   temperature > 0 (finite): the student logits and the teacher log-values
 *             are both divided by it and the loss is multiplied by its
 *             square (soft-target distillation); 1 is the method as described.
 *             Backward must get the same value as forward.
 *
 * Forward: loss, per-row log-sum-exp and per-row KL.
 *   loss     [1] fp32 device, written (mean KL over unmasked rows)
 *   lse      [n] fp32 device, written: LSE over the full vocabulary of each
 *            row's logits divided by the temperature (also for masked rows);
 *            pass it unchanged to bwd
 *   row_kl   [n] fp32 device or NULL: temperature^2 * KL_t (0 for masked rows)
 *   gathered [n, K] fp32 device or NULL: z_{t, i_{t,k}}, the raw student logit
 *            at each teacher id, taken from the same GEMM tiles that feed the
 *            log-sum-exp (undefined on masked rows and padding entries)
 *   workspace: device buffer of at least plan.fwd_workspace_bytes for the same
 *            (dtype, n, d, V, K, chunk); its contents need not be initialised.
 *            With chunk <= 0 the call itself picks the chunk: the planner's
 *            rule with this buffer's size as the budget, fitting the forward
 *            workspace only, so plan.fwd_workspace_bytes of an automatic plan
 *            always suffices (KD_E_WORKSPACE if not even chunk 256 fits).
 * The result does not depend on the chunk size (bitwise, for loss and lse).
 */
int kd_fused_chunked_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, float temperature, void* workspace,
                            size_t workspace_bytes, float* loss, float* lse, float* row_kl,
                            float* gathered, void* stream);

/*
 * Forward without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or evaluation loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and kernels as
 * kd_fused_chunked_kl_fwd, without the workspace: the call uses a scratch
 * array of KD_NOALLOC_SCRATCH_BYTES that the library holds in every GPU it
 * runs on until the process ends, and calls no hipMalloc, hipFree or other
 * allocating routine, nor creates events (kernel timing skips these calls).
 * With chunk <= 0 the largest automatic chunk whose forward workspace fits
 * the scratch is used; a problem whose forward workspace does not fit even at
 * chunk 256 (or at the chunk given) returns KD_E_WORKSPACE before any device
 * work (the 32K-token, 201088-vocabulary, K = 100 forward needs 126 MiB).
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind: calls that overlap on one GPU (several streams or host threads)
 * race and must be serialised by the caller.  The current device must be the
 * stream's.
 */
#define KD_NOALLOC_SCRATCH_BYTES (256ull << 20)
int kd_fused_chunked_kl_fwd_noalloc(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                                    const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                                    int64_t V, int32_t K, int64_t chunk, float temperature, float* loss,
                                    float* lse, float* row_kl, float* gathered, void* stream);

/*
 * Backward: recomputes each chunk's logits from H and W, forms G in registers
 * (rounded to the input dtype), then dH = G W and dW (+)= G^T H.
 *   lse       [n] fp32 device: exactly what kd_fused_chunked_kl_fwd wrote
 *   grad_loss [1] fp32 device: upstream gradient of the loss (1 for plain training)
 *   dH        [n, d] dtype device: OVERWRITTEN (rows of masked positions are 0)
 *   dW        [V, d] fp32 device: accumulate_dw != 0: ACCUMULATED (+=) into
 *             the caller's values; accumulate_dw == 0: OVERWRITTEN (every
 *             element written, prior contents never read, so it may be
 *             uninitialised)
 *   workspace: at least plan.bwd_workspace_bytes; with chunk <= 0 the chunk is
 *             picked as in the forward call, fitting the backward workspace.
 * No gradient is produced for the teacher inputs.
 */
int kd_fused_chunked_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, float temperature, const float* lse,
                            const float* grad_loss, void* dH, float* dW, int accumulate_dw,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Comparison variants: the two other ways the pages compute this same loss
 * (aib.vote summary, paragraph comparing Dense KL, Forward-chunked KL and
 * Fused chunked KL; Hugging Face blog "Making Knowledge Distillation Cheap
 * Enough to Run at Scale", sections "Two systems changes" and "Scaling to
 * long context lengths"), built to measure the fused calls against on the
 * same GPU.  They keep n x V fp32 grids, so their memory grows with n x V:
 *   dense KL:           the forward builds the student's full log-probability
 *                       grid log q [n, V] and the teacher's full probability
 *                       grid P [n, V] (p at the cached ids, 0 elsewhere) and
 *                       takes KL_t = sum_v P (log P - log q); the backward
 *                       forms G = gw (S_t exp(log q) - P) from the two grids;
 *   forward-chunked KL: the forward computes each chunk's logits, keeps them
 *                       all in a logit grid Z [n, V] and takes the loss with
 *                       the sparse teacher, as the fused forward does; the
 *                       backward forms G from the kept logits and the LSE
 *                       instead of recomputing them.
 * Both then run the fused backward's dH = G W and dW (+)= G^T H per chunk.
 * Arguments are those of the fused calls (temperature 1, bf16 H and W only:
 * KD_E_INVAL otherwise), plus the grid buffer: caller-owned device memory of
 * at least kd_comparator_grid_bytes(variant, n, V) bytes, 16-byte aligned,
 * written by the forward and read by the backward, which must get it
 * unchanged.  The workspace is the fused calls' (plan.fwd_workspace_bytes /
 * plan.bwd_workspace_bytes).  Results equal the fused calls' up to rounding,
 * except that the dense grid sums an id a row repeats before taking its
 * entropy term p log p (the sparse form keeps one term per entry).
 */
enum { KD_VARIANT_DENSE = 1, KD_VARIANT_FORWARD_CHUNKED = 2 };
/* Bytes of the grid buffer (dense: 2 grids, forward-chunked: 1); 0 for bad arguments. */
size_t kd_comparator_grid_bytes(int variant, int64_t n, int64_t V);
int kd_dense_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logp,
                    const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk, void* grid,
                    size_t grid_bytes, void* workspace, size_t workspace_bytes, float* loss, float* lse,
                    float* row_kl, void* stream);
int kd_dense_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logp,
                    const uint8_t* mask, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                    const void* grid, size_t grid_bytes, const float* lse, const float* grad_loss, void* dH,
                    float* dW, int accumulate_dw, void* workspace, size_t workspace_bytes, void* stream);
int kd_forward_chunked_kl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                              const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V,
                              int32_t K, int64_t chunk, void* grid, size_t grid_bytes, void* workspace,
                              size_t workspace_bytes, float* loss, float* lse, float* row_kl, void* stream);
int kd_forward_chunked_kl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                              const float* topk_logp, const uint8_t* mask, int64_t n, int64_t d, int64_t V,
                              int32_t K, int64_t chunk, const void* grid, size_t grid_bytes, const float* lse,
                              const float* grad_loss, void* dH, float* dW, int accumulate_dw, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Teacher top-K cache builder: the offline cache the loss above consumes.
 * The pages keep, for every position, the K most likely tokens of the
 * teacher, computed once (Hugging Face blog "Making Knowledge Distillation
 * Cheap Enough to Run at Scale", section "Two systems changes"; aimodeling.com
 * article, section "First cut: remove the teacher from the training loop").
 * For every row t of the teacher's final hidden states:
 *   z_{t,v} = Ht[t] . Wt[v]  (fp32 accumulation of dtype products)
 *   topk_idx[t, :]  the K ids with the largest z_{t,v}, in decreasing order of
 *                   z; equal logits are taken in increasing id order
 *   topk_logp[t, :] z_{t,v} - LSE_v(z_t) at those ids (full-vocabulary
 *                   log-probabilities: the format of topk_idx / topk_logp of
 *                   the loss calls)
 * No row's logits are ever stored: each chunk of rows runs the output GEMM
 * twice, once for LSE and per-tile maxima (the K-th largest tile maximum is a
 * threshold that every top-K logit reaches), once to collect the logits at or
 * above the threshold into a per-row list of at most `cap` entries.
 *
 * Plan: chunk as for kd_plan_query (<= 0: the planner picks the largest that
 * fits hbm_budget, 0 = half the free device memory); cap <= 0 picks
 * min(V, 4096), or V when V has fewer than K 256-wide tiles; cap >= K.
 */
typedef struct kd_topk_plan {
  int64_t chunk;
  int64_t n_chunks;
  int64_t cap;              /* candidate-list entries per row */
  int64_t vocab_tiles;
  size_t workspace_bytes;   /* needed by kd_teacher_topk */
} kd_topk_plan_t;

int kd_teacher_topk_plan(int dtype, int64_t n, int64_t d, int64_t V, int32_t K, int64_t chunk,
                         int64_t cap, size_t hbm_budget, kd_topk_plan_t* out);

/*
 *   Ht        [n, d]  dtype device   teacher hidden states (16-byte aligned)
 *   Wt        [V, d]  dtype device   teacher output-projection weight
 *   K         1 <= K <= min(V, 4096)
 *   topk_idx  [n, K]  int32 device, written
 *   topk_logp [n, K]  fp32 device, written
 *   workspace device buffer of at least plan.workspace_bytes (uninitialised)
 * Unlike the loss calls this one synchronises `stream` before returning: it
 * returns KD_E_RANGE if some row had more than cap logits at or above its
 * threshold (only for rows of nearly constant logits); those rows' entries are
 * then incomplete and the call should be repeated with a larger cap.  NaN
 * logits are unsupported (such a row may come back with ids of -1).
 */
int kd_teacher_topk(int dtype, const void* Ht, const void* Wt, int64_t n, int64_t d, int64_t V,
                    int32_t K, int64_t chunk, int64_t cap, void* workspace, size_t workspace_bytes,
                    int32_t* topk_idx, float* topk_logp, void* stream);

/* Human-readable name of a status code (static storage). */
const char* kd_status_string(int status);

/* Message of the last failing call on this host thread ("" if none). */
const char* kd_last_error_message(void);

/*
 * Validation mode (off by default; the environment variable KDLOSS_VALIDATE=1
 * switches it on at load time).  When on, fwd and bwd synchronise the stream
 * after teacher preparation and return KD_E_RANGE if an unmasked row holds an
 * id outside [0, V).  When off such ids are skipped (their terms are missing
 * and gathered values are left unwritten) but never read out of bounds.
 */
int kd_set_validate(int on);

/*
 * Kernel timing.  While enabled, every kernel launch is bracketed by two HIP
 * events recorded on the call's stream; kd_profile_read synchronises on the
 * recorded events and returns, per kernel class, the launch count, the summed
 * event-to-event time, and the algorithmic flops and bytes of those launches.
 * The records are kept per process and are not thread-safe.
 */
typedef struct kd_kernel_stat {
  char name[48];
  int64_t launches;
  double total_ms;
  double flops;   /* algorithmic: 2*M*N*K for the contractions, 0 otherwise */
  double bytes;   /* algorithmic HBM bytes (operands read once, outputs written once) */
} kd_kernel_stat_t;

int kd_profile_enable(int on);
int kd_profile_reset(void);
int kd_profile_read(kd_kernel_stat_t* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* KDLOSS_H */
