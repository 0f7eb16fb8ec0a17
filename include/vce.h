/*
 * libvce: fused cross-entropy over a large vocabulary for AMD MI355X (gfx950).
 *
 * Two forms of the same loss are exported.
 *
 *  1. Logits cross-entropy (ce_forward / ce_backward).  The operation is the
 *     one of the TransformerEngine cross-entropy API page (Signature and I/O
 *     Contract): logits of shape (B,SQ,V) or (SQ,B,V), integer targets of
 *     shape (B,SQ) or (SQ,B), label smoothing, an optional averaged scalar
 *     loss, an ignore index (default -100), loss in FP32 computed in FP32
 *     whatever the input dtype (Description).  As in the TransformerEngine
 *     PR "Minimize the memory usage of the fused cross entropy kernel"
 *     (Changes; Sequence Diagram), the forward saves per-row statistics only,
 *     the backward rebuilds the gradient from them, and the backward may write
 *     the gradient over the logits ("overwrite_input", destructive reuse).
 *
 *  2. Fused linear cross-entropy (lce_forward / lce_backward).  The loss of
 *     logits = X W^T computed tile by tile without storing the (M, V) logit
 *     matrix: the cut-cross-entropy package description (linear_cross_entropy
 *     of embeddings, classifier and labels) and the Liger-Kernel PR "Add SM100
 *     tensor-parallel fused scaled cross entropy" (Summary: classifier GEMM
 *     fused with NLL/LSE; Backward: dZ from recomputed logits, then dX and dW;
 *     a caller-owned reusable workspace with a size query).
 *
 * Definitions (per row r with logits z, target t, smoothing eps, vocabulary V):
 *     m = max_v z_v,  d = sum_v exp(z_v - m),  lse = m + ln d
 *     q_v = (1 - eps) [v = t] + eps / V        (eps/V on every class)
 *     loss_r = -sum_v q_v (z_v - lse) = (1-eps)(lse - z_t) + eps (lse - mean_v z_v)
 *     grad[r, v] = g_r (exp(z_v - lse) - q_v)
 *   g_r = grad_output[r] for per-token loss, grad_output[0] / n_valid for the
 *   averaged loss.  Rows whose target equals ignore_idx have loss 0 and
 *   gradient 0 and are excluded from the average (numerator and count).  With
 *   no valid row the average is 0 (count taken as 1).  A target that is
 *   neither ignore_idx nor in [0, V) yields NaN loss and NaN gradient for that
 *   row (it cannot be reported without a device synchronisation).
 *
 * Saved statistics: stats is (N, 4) FP32 per row = (m, d, z_t, mean_v z_v),
 * 16 bytes per row.  Rows that are ignored hold zeros there.
 *
 * Value range: logits are read as IEEE values.  -inf entries (padded
 * vocabularies) get probability 0, and so do entries masked with a finite
 * value far below the row's maximum (such as -FLT_MAX); with eps > 0 the
 * mean logit enters the loss, and it is an FP32 sum that overflows when many
 * logits lie near +-FLT_MAX.  A row whose largest logit exceeds 2^30 in
 * magnitude is outside the logits forward's exponent form (its statistics
 * are not meaningful), as are linear-form logits beyond about 2^29.
 *
 * Entropy (optional, the "optional entropy" output of the Liger-Kernel PR,
 * Summary): H_r = -sum_v p_v ln p_v of p = softmax(z_r), FP32 per row, 0 for
 * ignored rows (it does not depend on the target otherwise).  Given an
 * upstream gradient gH of the entropy, the backward adds
 *     gH_r dH/dz_v = gH_r p_v (E_p[z] - z_v),   E_p[z] = lse_r - H_r,
 * to the loss gradient; it reads H_r from the forward's entropy output.
 *
 * Conventions for every entry point:
 *  - All pointers are DEVICE pointers on the current HIP device, owned by
 *    the caller.  The library never allocates, frees or synchronises and
 *    keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  All work
 *    is enqueued on it in order, so a call is safe inside HIP graph capture.
 *  - Return value 0 means every kernel was enqueued.  A nonzero VCE_E* code
 *    means the arguments were rejected and nothing was launched (VCE_EHIP: a
 *    launch failed).  vce_strerror() names a code.
 *  - N = d0 * d1 rows; N = 0 is a successful no-op (with reduce_loss the
 *    averaged loss 0 and count 0 are still written).
 */
#ifndef VCE_H
#define VCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vce_status {
  VCE_OK = 0,
  VCE_EINVAL = 1,       /* null pointer, bad size, eps outside [0,1], negative stride */
  VCE_EDTYPE = 2,       /* dtype not VCE_DTYPE_FP32 / VCE_DTYPE_BF16 */
  VCE_EALIGN = 3,       /* pointer or stride not aligned as required */
  VCE_EALIAS = 4,       /* overwrite_input set but grad != logits, or buffers overlap */
  VCE_EWORKSPACE = 5,   /* workspace too small (see lce_workspace_size) */
  VCE_EHIP = 6,         /* a kernel launch failed */
  VCE_EUNSUPPORTED = 7, /* a size the library does not handle (see the entry point) */
  VCE_ESCRATCH = 8      /* beyond the static scratch of lce_forward_noalloc */
};

enum vce_dtype { VCE_DTYPE_FP32 = 0, VCE_DTYPE_BF16 = 1 };

/* Text for a status code (static storage). */
const char* vce_strerror(int status);

/*
 * ce_forward: single-pass online-softmax forward of logits cross-entropy.
 *
 *  logits   (d0, d1, V) elements of `dtype` (FP32 or BF16).  Row (i0, i1)
 *           starts at element i0*ls0 + i1*ls1; the V elements of a row are
 *           contiguous.  (B,SQ,V) storage: d0=B, d1=SQ; (SQ,B,V): d0=SQ, d1=B;
 *           any permuted view works through the two strides.  Must be aligned
 *           to the element size.
 *  targets  int64, element (i0, i1) at i0*ts0 + i1*ts1.
 *  label_smoothing  eps in [0, 1].   reduce_loss  0 or 1.
 *  ignore_idx       rows with this target are ignored (may lie in [0, V)).
 *  loss_tok (N) FP32, always written, flattened row order r = i0*d1 + i1.
 *  loss_mean  1 FP32: written iff reduce_loss (may be NULL otherwise).
 *  stats    (N, 4) FP32 saved statistics (see above), always written.
 *  n_valid  1 int32: count of non-ignored rows; required iff reduce_loss
 *           (the backward of the averaged loss reads it), else may be NULL.
 *  Kernels: one row sweep (one workgroup per row: 512 threads, 256 for rows
 *  of at most 48 KB), plus one single-workgroup deterministic mean when
 *  reduce_loss or n_valid is given.
 *  entropy  (N) FP32, or NULL: written iff non-NULL (costs one more FMA per
 *           logit; the path without it is unchanged).
 */
int ce_forward(const void* logits, int dtype, int64_t d0, int64_t d1, int64_t V,
               int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
               float label_smoothing, int reduce_loss, int64_t ignore_idx,
               float* loss_tok, float* loss_mean, float* stats, int32_t* n_valid,
               float* entropy, void* stream);

/*
 * ce_backward: rebuild the logits gradient from the saved statistics.
 *
 *  logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1, label_smoothing,
 *  reduce_loss, ignore_idx: exactly as given to ce_forward.
 *  grad     gradient, same dtype, shape and strides as logits (FP32 math,
 *           stored rounded to nearest even for BF16).  Every element of every
 *           row is written (ignored rows: zeros).
 *  stats    (N, 4) from ce_forward.   n_valid: from ce_forward; read iff
 *           reduce_loss.
 *  grad_output  FP32: 1 element if reduce_loss, else (N) in flattened row
 *           order.
 *  overwrite_input  nonzero: grad must equal logits, and the logits are
 *           replaced by the gradient (no extra buffer).  Zero: grad and
 *           logits must not overlap (VCE_EALIAS otherwise).
 *  entropy, grad_entropy  (N) FP32 each, or NULL: with grad_entropy the
 *           gradient also gets grad_entropy[r] dH/dz (see above), entropy being
 *           the forward's entropy output (required then).
 */
int ce_backward(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1, int64_t V,
                int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
                const float* stats, const int32_t* n_valid, const float* grad_output,
                const float* entropy, const float* grad_entropy, float label_smoothing,
                int reduce_loss, int64_t ignore_idx, int overwrite_input, void* stream);

/*
 * ce_forward_backward: ce_forward and ce_backward in one call, for a loss whose
 * upstream gradient is known when the loss is asked for (the loss is the last
 * operation, e.g. grad_output = 1).  The outputs are those of ce_forward
 * followed by ce_backward with the same arguments (no entropy), bit for bit;
 * the logits are read once instead of twice: each row is held on chip between
 * its statistics and its gradient (rows of up to 256 KB: 131072 BF16 or 65536
 * FP32 logits, at most; longer rows take the two sweeps inside this call).  The
 * flow the TransformerEngine PR replaced also formed the derivative in the
 * forward (Changes), as an FP32 buffer for a later multiply by the incoming
 * gradient; here grad_output is applied at once and the gradient is stored in
 * the input dtype, in a separate buffer or over the logits.
 *
 *  Arguments as in ce_forward and ce_backward; loss_tok, loss_mean, stats,
 *  n_valid are written as ce_forward writes them, grad as ce_backward does.
 */
int ce_forward_backward(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1,
                        int64_t V, int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0,
                        int64_t ts1, const float* grad_output, float label_smoothing,
                        int reduce_loss, int64_t ignore_idx, int overwrite_input,
                        float* loss_tok, float* loss_mean, float* stats, int32_t* n_valid,
                        void* stream);

/*
 * Vocabulary-sharded logits cross-entropy.  The per-shard half of the
 * tensor-parallel flow of the TransformerEngine PR "Minimize the memory usage
 * of the fused cross entropy kernel" (Changes: the multi-GPU path with two
 * kernels; Sequence Diagram: local statistics, all-gather, global statistics).
 * Shard k holds vocabulary columns [vocab_start_k, vocab_start_k + V_local_k)
 * of a V-column vocabulary.  The exchange between shards is the caller's:
 * one process per shard gathers the partials of every shard (e.g. an
 * all-gather of N x 16 bytes each) and calls ce_merge_shards, which runs the
 * same on every shard.  The backward is then local to each shard.
 *
 *  ce_forward_shard: partial (N, 4) FP32 per row = (m_k, d_k, sum_v z_v,
 *    z_t if vocab_start <= t < vocab_start + V_local else 0) over the shard's
 *    columns; ignored rows hold zeros.  logits, dtype, d0, d1, ls0, ls1,
 *    targets, ts0, ts1, ignore_idx as in ce_forward with V = V_local; targets
 *    are indices into the full vocabulary.  partial: 16-byte aligned.
 *    partial_w (N) FP32 or NULL: when given, also the shard's entropy
 *    statistic w_k = sum_v exp(z_v - m_k) (z_v - m_k) / ln 2 (0 for ignored
 *    rows), for the entropy output of ce_merge_shards (the Liger-Kernel PR's
 *    tensor-parallel forward offers the entropy, Summary).
 */
int ce_forward_shard(const void* logits, int dtype, int64_t d0, int64_t d1, int64_t V_local,
                     int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
                     int64_t vocab_start, int64_t ignore_idx, float* partial, float* partial_w,
                     void* stream);

/*
 *  ce_merge_shards: partials (n_shards, N, 4), the shards' partial outputs
 *    stacked in a fixed order (the result is bitwise the same on every
 *    process given the same order).  Merges m = max_k m_k, d = sum_k d_k
 *    exp(m_k - m), sum z and z_t, and writes loss_tok, loss_mean, stats and
 *    n_valid exactly as ce_forward would for the whole (N, V) logits, the
 *    label smoothing eps / V and the mean logit taken over the full V.  A
 *    target neither ignore_idx nor in [0, V) gives NaN, as in ce_forward.
 *    entropy (N) FP32 or NULL: when given, the per-row entropy of the full
 *    row, as ce_forward's, from partials_w (n_shards, N), the shards'
 *    partial_w outputs in the same order (required then; otherwise unread):
 *    W = sum_k exp(m_k - m) (ln 2 w_k + d_k (m_k - m)), H = ln d - W / d.
 */
int ce_merge_shards(const float* partials, const float* partials_w, int64_t n_shards, int64_t d0,
                    int64_t d1, const int64_t* targets, int64_t ts0, int64_t ts1, int64_t V,
                    float label_smoothing, int reduce_loss, int64_t ignore_idx, float* loss_tok,
                    float* loss_mean, float* stats, int32_t* n_valid, float* entropy,
                    void* stream);

/*
 *  ce_backward_shard: ce_backward for the shard's columns of the gradient,
 *    from the merged stats and n_valid of ce_merge_shards: V is the full
 *    vocabulary (vocab_start + V_local <= V), and only the shard holding the
 *    target subtracts (1 - eps) g there.  entropy, grad_entropy: the merged
 *    entropy of ce_merge_shards and its upstream gradient, as in ce_backward.
 *    Other arguments as in ce_backward.
 */
int ce_backward_shard(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1,
                      int64_t V_local, int64_t ls0, int64_t ls1, const int64_t* targets,
                      int64_t ts0, int64_t ts1, int64_t vocab_start, int64_t V,
                      const float* stats, const int32_t* n_valid, const float* grad_output,
                      const float* entropy, const float* grad_entropy, float label_smoothing,
                      int reduce_loss, int64_t ignore_idx, int overwrite_input, void* stream);

/*
 * vce_shift_targets: causal label shift, the optional token shifting of the
 * cut-cross-entropy package description (what_it_does: shifting for causal
 * language modelling): position s of a sequence is scored against the label
 * of position s + 1, and the last position of every sequence has no label.
 *
 *  targets  int64 (d0, d1), element (i0, i1) at i0*ts0 + i1*ts1 (as given to
 *           the other entry points).
 *  seq_axis 0: the sequence runs along d0 ((SQ,B) storage); 1: along d1
 *           ((B,SQ) storage, or (1, M) for the flattened tokens of one
 *           sequence).
 *  shifted  int64 (d0, d1) contiguous, flattened row order r = i0*d1 + i1,
 *           8-byte aligned, must not overlap targets: shifted(i0, i1) =
 *           targets(i0 + 1, i1) (seq_axis 0) or targets(i0, i1 + 1) (seq_axis 1),
 *           and ignore_idx at the last position.  Pass it (strides d1, 1) as the
 *           targets of any other entry point: the last positions are then
 *           ignored rows (loss 0, excluded from the mean, zero gradient).
 */
int vce_shift_targets(const int64_t* targets, int64_t d0, int64_t d1, int64_t ts0, int64_t ts1,
                      int seq_axis, int64_t ignore_idx, int64_t* shifted, void* stream);

/*
 * lce_workspace_size: bytes of device workspace lce_forward and lce_backward
 * need for an (M, H, V) problem (one buffer serves both; its contents need
 * not survive between calls).  Analogue of the workspace query API of the
 * Liger-Kernel PR (Summary).  Returns 0 for invalid sizes.
 */
size_t lce_workspace_size(int64_t M, int64_t H, int64_t V);

/*
 * lce_forward: loss of logits = X W^T without storing the logits.
 *
 *  X (M, H) and W (V, H): BF16, row-major, contiguous, 16-byte aligned;
 *  H must be a multiple of 8 (VCE_EUNSUPPORTED otherwise).  FP32
 *  accumulation on the matrix cores.
 *  targets (M) int64 contiguous.   Outputs as ce_forward with N = M:
 *  loss_tok (M), loss_mean (iff reduce_loss), stats (M, 4), n_valid.
 *  entropy (M) FP32 or NULL, as in ce_forward.
 *  workspace: at least lce_workspace_size(M, H, V) bytes, 256-byte aligned.
 */
int lce_forward(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                const int64_t* targets, float label_smoothing, int reduce_loss,
                int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                int32_t* n_valid, float* entropy, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * lce_forward_noalloc: lce_forward without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs
 * and kernels as lce_forward (BF16 X and W), bit for bit the same results;
 * the forward's per-tile partials live in a static device array of the
 * library, LCE_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held from the
 * library's first use on a device until the process ends.  That bounds the
 * problem: 16 * ceil(V / 256) * Mp + 4 * Mp bytes, Mp = M rounded up to a
 * multiple of 256, must fit (M = 4096, V = 131072 takes 32 MiB; M = 4096
 * fits V up to 261888); larger problems return VCE_ESCRATCH and launch
 * nothing.  Nothing in the scratch
 * needs to start at zero.  Every call on one device shares its scratch:
 * calls that may overlap on one device (concurrent streams, graphs replayed
 * on other streams) race and must be serialised by the caller.  The device
 * is the stream's own (the current device for the NULL stream); no call
 * allocates, frees or synchronises.
 */
#define LCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lce_forward_noalloc(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                        const int64_t* targets, float label_smoothing, int reduce_loss,
                        int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                        int32_t* n_valid, float* entropy, void* stream);

/*
 * lce_backward: dX (M, H) and dW (V, H), BF16, overwritten (not accumulated).
 *
 *  X, W, M, H, V, targets, label_smoothing, reduce_loss, ignore_idx: as given
 *  to lce_forward.  stats, n_valid: from lce_forward.  grad_output: FP32, 1
 *  element if reduce_loss else (M).  The logits are recomputed chunk by chunk
 *  over the vocabulary; the gradient of each chunk is held in the workspace.
 *  entropy, grad_entropy: as in ce_backward.  With M = 0, dW is set to zero
 *  (X, targets and the workspace are not read).
 */
int lce_backward(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                 const int64_t* targets, const float* stats, const int32_t* n_valid,
                 const float* grad_output, const float* entropy, const float* grad_entropy,
                 float label_smoothing, int reduce_loss, int64_t ignore_idx, void* dX, void* dW,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scaled linear form (the Liger-Kernel PR "Add SM100 tensor-parallel fused
 * scaled cross entropy", title and Summary: a "fused scaled linear
 * cross-entropy"; the pages do not say what is scaled).  Read here as the
 * loss of logits = logit_scale * X W^T, a positive scalar applied to the
 * logits before the softmax (a logit scale or inverse temperature):
 *     loss_r = CE(logit_scale * (X W^T)_r, t_r), with eps and ignore_idx as
 *     in lce_forward;
 * dX and dW are the gradients of that loss (logit_scale times the gradient
 * with respect to the scaled logits, pushed through X W^T).  The saved
 * statistics and the entropy are those of the scaled logits.
 *
 *  lce_forward_scaled, lce_backward_scaled: the arguments of lce_forward and
 *    lce_backward plus logit_scale, which must be finite and > 0
 *    (VCE_EINVAL otherwise, nothing launched); the same backward must get
 *    the same logit_scale as its forward.  logit_scale = 1 gives bit for bit
 *    the results of lce_forward and lce_backward; a power of two 2^k gives
 *    bit for bit the unscaled results for W * 2^k (dW then 2^k times the
 *    unscaled dW, as the chain rule says).  The scale is folded into the
 *    exponent's factor and the gradient's factor, so it costs no work per
 *    logit.
 */
int lce_forward_scaled(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                       float logit_scale, const int64_t* targets, float label_smoothing,
                       int reduce_loss, int64_t ignore_idx, float* loss_tok, float* loss_mean,
                       float* stats, int32_t* n_valid, float* entropy, void* workspace,
                       size_t workspace_bytes, void* stream);
int lce_backward_scaled(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                        float logit_scale, const int64_t* targets, const float* stats,
                        const int32_t* n_valid, const float* grad_output, const float* entropy,
                        const float* grad_entropy, float label_smoothing, int reduce_loss,
                        int64_t ignore_idx, void* dX, void* dW, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * FP32 inputs to the linear form (the cross-entropy API page, Description:
 * BF16 or FP32 input, FP32 loss and gradient computation).  X (M, H) and W
 * (V, H) are FP32, row-major, contiguous, 16-byte aligned, H a multiple of 8.
 * The matrix cores take each operand as two BF16 planes, x = hi + lo with
 * hi = bf16(x) and lo = bf16(x - hi) (round to nearest even: hi + lo is x to
 * within 2^-16 of its size), and every product as hi*hi + hi*lo + lo*hi with
 * FP32 accumulation: each product is off by at most about 3 * 2^-16 of its
 * size, for three times the BF16 matrix-core work.  The gradient dZ is split
 * the same way before the dX and dW products.
 *
 *  lce_workspace_size_f32: bytes of workspace for an (M, H, V) problem (the
 *    BF16 planes of X and W, 4 (M + V) H bytes, plus what the BF16 form
 *    needs, with dZ in two planes); 0 for invalid sizes.
 *  lce_forward_f32: as lce_forward (all outputs FP32, same layouts).
 *  lce_backward_f32: as lce_backward, with dX (M, H) and dW (V, H) FP32,
 *    overwritten.  Each call splits X and W again (the workspace need not
 *    survive from the forward).
 */
size_t lce_workspace_size_f32(int64_t M, int64_t H, int64_t V);

int lce_forward_f32(const float* X, const float* W, int64_t M, int64_t H, int64_t V,
                    const int64_t* targets, float label_smoothing, int reduce_loss,
                    int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                    int32_t* n_valid, float* entropy, void* workspace, size_t workspace_bytes,
                    void* stream);

int lce_backward_f32(const float* X, const float* W, int64_t M, int64_t H, int64_t V,
                     const int64_t* targets, const float* stats, const int32_t* n_valid,
                     const float* grad_output, const float* entropy, const float* grad_entropy,
                     float label_smoothing, int reduce_loss, int64_t ignore_idx, float* dX,
                     float* dW, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Vocabulary-sharded linear cross-entropy: the per-shard half of the
 * tensor-parallel forward of the Liger-Kernel PR (Summary: tensor-parallel
 * fused linear cross-entropy; the classifier W sharded by vocabulary rows),
 * with the same partial statistics as ce_forward_shard, so ce_merge_shards
 * merges them.  W_local (V_local, H) holds vocabulary rows
 * [vocab_start, vocab_start + V_local) of the full classifier.  The
 * workspace is sized by lce_workspace_size(M, H, V_local).
 *
 *  lce_forward_shard: partial (M, 4) FP32 and optional partial_w (M) as in
 *    ce_forward_shard, for the logits X W_local^T, which are never stored.
 *    Other arguments as in lce_forward.
 */
int lce_forward_shard(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                      const int64_t* targets, int64_t vocab_start, int64_t ignore_idx,
                      float* partial, float* partial_w, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 *  lce_backward_shard: from the merged stats and n_valid (ce_merge_shards
 *    over every shard, V the full vocabulary), dW_local (V_local, H) of this
 *    shard and this shard's share of dX, dZ_k W_local (M, H): the full dX is
 *    the sum of the shards' shares (the caller's reduction across shards).
 *    BF16 outputs, overwritten.  entropy, grad_entropy: the merged entropy
 *    and its upstream gradient, as in ce_backward_shard.  Other arguments as
 *    in lce_backward.
 */
int lce_backward_shard(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                       const int64_t* targets, int64_t vocab_start, int64_t V,
                       const float* stats, const int32_t* n_valid, const float* grad_output,
                       const float* entropy, const float* grad_entropy, float label_smoothing,
                       int reduce_loss, int64_t ignore_idx, void* dX, void* dW, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Tensor-parallel scaled linear cross-entropy, the combination the
 * Liger-Kernel PR "Add SM100 tensor-parallel fused scaled cross entropy"
 * names in its title and Summary: the shard forms above for the logits
 * logit_scale * X W_local^T (the scaled form of lce_forward_scaled).  Every
 * shard of one problem takes the same logit_scale.  The partials are those of
 * the scaled logits, so ce_merge_shards merges them unchanged; the backward
 * takes the merged statistics and the same logit_scale.
 *
 *  lce_forward_shard_scaled, lce_backward_shard_scaled: the arguments of
 *    lce_forward_shard and lce_backward_shard plus logit_scale, finite and
 *    > 0 (VCE_EINVAL otherwise, nothing launched).  logit_scale = 1 gives bit
 *    for bit the unscaled shard results; 2^k those of the unscaled shard
 *    forms for W_local * 2^k.
 */
int lce_forward_shard_scaled(const void* X, const void* W, int64_t M, int64_t H,
                             int64_t V_local, float logit_scale, const int64_t* targets,
                             int64_t vocab_start, int64_t ignore_idx, float* partial,
                             float* partial_w, void* workspace, size_t workspace_bytes,
                             void* stream);
int lce_backward_shard_scaled(const void* X, const void* W, int64_t M, int64_t H,
                              int64_t V_local, float logit_scale, const int64_t* targets,
                              int64_t vocab_start, int64_t V, const float* stats,
                              const int32_t* n_valid, const float* grad_output,
                              const float* entropy, const float* grad_entropy,
                              float label_smoothing, int reduce_loss, int64_t ignore_idx,
                              void* dX, void* dW, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * vce_gemm_bf16: the matrix-core building block of the linear form, exported
 * so it can be checked and timed on its own, as the Liger-Kernel PR "Add SM100
 * tensor-parallel fused scaled cross entropy" validates its classifier GEMM
 * apart from the fused loss (SM90 regression validation: standalone forward
 * GEMM numerical cases).  C (rows, cols) FP32 row-major
 * with leading dimension ldc:  C[i][j] = sum_k P(i, k) Q(j, k), BF16 operands,
 * FP32 accumulation.  Each operand is stored
 *   K-contiguous   (p_dim / q_dim = 0): P(i, k) = P[i * ldp + k]
 *   dim-contiguous (p_dim / q_dim = 1): P(i, k) = P[k * ldp + i]
 * (likewise Q with j, ldq).  The contiguous axis must be a multiple of 8 long
 * (K for a K-contiguous operand, rows / cols for a dim-contiguous one); ldp,
 * ldq multiples of 8 and at most 2^22; P and Q 16-byte aligned.  The backward
 * of the linear form uses all three layout pairs it needs through this core.
 */
int vce_gemm_bf16(const void* P, int64_t ldp, int p_dim, const void* Q, int64_t ldq, int q_dim,
                  int64_t rows, int64_t cols, int64_t K, float* C, int64_t ldc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VCE_H */
