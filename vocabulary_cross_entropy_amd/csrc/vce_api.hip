// C-ABI of libvce: argument validation and kernel dispatch.  Declarations and
// the contract of every entry point are in include/vce.h.
//
// Nothing here allocates, frees or synchronises: each entry point checks its
// arguments on the host, then enqueues its kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "vce.h"
#include "vce_internal.h"

namespace {

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? VCE_OK : VCE_EHIP; }

// Byte extent [lo, hi) touched by a (d0, d1, V) strided tensor.
inline void extent(const void* base, int64_t d0, int64_t d1, int64_t V, int64_t s0, int64_t s1,
                   int64_t es, uintptr_t* lo, uintptr_t* hi) {
  const int64_t last = (d0 - 1) * s0 + (d1 - 1) * s1 + V;
  *lo = reinterpret_cast<uintptr_t>(base);
  *hi = *lo + (uintptr_t)(last * es);
}

struct CeShape {
  int64_t N;
  int64_t es;
};

int check_ce_common(const void* logits, int dtype, int64_t d0, int64_t d1, int64_t V, int64_t ls0,
                    int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1, float eps,
                    int reduce_loss, CeShape* sh) {
  if (dtype != VCE_DTYPE_FP32 && dtype != VCE_DTYPE_BF16) return VCE_EDTYPE;
  if (d0 < 0 || d1 < 0 || V <= 0) return VCE_EINVAL;
  if (ls0 < 0 || ls1 < 0 || ts0 < 0 || ts1 < 0) return VCE_EINVAL;
  if (!(eps >= 0.0f && eps <= 1.0f)) return VCE_EINVAL;  // also rejects NaN
  if (reduce_loss != 0 && reduce_loss != 1) return VCE_EINVAL;
  int64_t N;
  if (!mul_ok(d0, d1, &N) || N > (int64_t)INT32_MAX) return VCE_EINVAL;
  const int64_t es = dtype == VCE_DTYPE_FP32 ? 4 : 2;
  if (N > 0) {
    if (!logits || !targets) return VCE_EINVAL;
    int64_t span0, span1, tmp;
    if (!mul_ok(d0 - 1, ls0, &span0) || !mul_ok(d1 - 1, ls1, &span1)) return VCE_EINVAL;
    if (span0 > INT64_MAX / 8 - span1 - V || !mul_ok(span0 + span1 + V, es, &tmp))
      return VCE_EINVAL;
    if (!aligned(logits, (size_t)es) || !aligned(targets, 8)) return VCE_EALIGN;
  }
  sh->N = N;
  sh->es = es;
  return VCE_OK;
}

}  // namespace

extern "C" {

const char* vce_strerror(int status) {
  switch (status) {
    case VCE_OK: return "success";
    case VCE_EINVAL: return "invalid argument (null pointer, size, stride or label_smoothing)";
    case VCE_EDTYPE: return "unsupported dtype (expected FP32 or BF16)";
    case VCE_EALIGN: return "misaligned pointer or stride";
    case VCE_EALIAS: return "buffer aliasing violates overwrite_input";
    case VCE_EWORKSPACE: return "workspace too small";
    case VCE_EHIP: return "HIP kernel launch failed";
    case VCE_EUNSUPPORTED: return "size not supported by the library";
    case VCE_ESCRATCH:
      return "problem larger than the static scratch of lce_forward_noalloc "
             "(LCE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int ce_forward(const void* logits, int dtype, int64_t d0, int64_t d1, int64_t V, int64_t ls0,
               int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
               float label_smoothing, int reduce_loss, int64_t ignore_idx, float* loss_tok,
               float* loss_mean, float* stats, int32_t* n_valid, float* entropy, void* stream) {
  CeShape sh;
  int rc = check_ce_common(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1,
                           label_smoothing, reduce_loss, &sh);
  if (rc != VCE_OK) return rc;
  if (reduce_loss && (!loss_mean || !n_valid)) return VCE_EINVAL;
  if (sh.N > 0 && (!loss_tok || !stats)) return VCE_EINVAL;
  if (stats && !aligned(stats, 16)) return VCE_EALIGN;
  if ((loss_tok && !aligned(loss_tok, 4)) || (loss_mean && !aligned(loss_mean, 4)) ||
      (n_valid && !aligned(n_valid, 4)) || (entropy && !aligned(entropy, 4)))
    return VCE_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);

  vce::CeFwdParams p;
  p.logits = logits;
  p.d1 = d1 > 0 ? d1 : 1;
  p.ls0 = ls0;
  p.ls1 = ls1;
  p.V = V;
  p.targets = targets;
  p.ts0 = ts0;
  p.ts1 = ts1;
  p.eps = label_smoothing;
  p.ignore_idx = ignore_idx;
  p.loss_tok = loss_tok;
  p.stats = stats;
  p.entropy = entropy;
  p.v0 = 0;
  p.partial = nullptr;
  p.partial_w = nullptr;
  rc = launch_status(vce::launch_ce_forward(p, dtype, sh.N, s));
  if (rc != VCE_OK) return rc;
  if (reduce_loss || n_valid) {
    vce::CeMeanParams mp;
    mp.loss_tok = loss_tok;
    mp.targets = targets;
    mp.N = sh.N;
    mp.d1 = d1 > 0 ? d1 : 1;
    mp.ts0 = ts0;
    mp.ts1 = ts1;
    mp.ignore_idx = ignore_idx;
    mp.loss_mean = reduce_loss ? loss_mean : nullptr;
    mp.n_valid = n_valid;
    rc = launch_status(vce::launch_ce_mean(mp, s));
  }
  return rc;
}

int ce_backward(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1, int64_t V,
                int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
                const float* stats, const int32_t* n_valid, const float* grad_output,
                const float* entropy, const float* grad_entropy, float label_smoothing,
                int reduce_loss, int64_t ignore_idx, int overwrite_input, void* stream) {
  CeShape sh;
  int rc = check_ce_common(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1,
                           label_smoothing, reduce_loss, &sh);
  if (rc != VCE_OK) return rc;
  if (overwrite_input != 0 && overwrite_input != 1) return VCE_EINVAL;
  if (sh.N == 0) return VCE_OK;
  if (!grad || !stats || !grad_output || (reduce_loss && !n_valid)) return VCE_EINVAL;
  if (grad_entropy && !entropy) return VCE_EINVAL;
  if (!aligned(stats, 16) || !aligned(grad_output, 4) || (n_valid && !aligned(n_valid, 4)) ||
      (entropy && !aligned(entropy, 4)) || (grad_entropy && !aligned(grad_entropy, 4)))
    return VCE_EALIGN;
  if (overwrite_input) {
    if (grad != logits) return VCE_EALIAS;
  } else {
    uintptr_t a0, a1, b0, b1;
    extent(logits, d0, d1, V, ls0, ls1, sh.es, &a0, &a1);
    extent(grad, d0, d1, V, ls0, ls1, sh.es, &b0, &b1);
    if (a0 < b1 && b0 < a1) return VCE_EALIAS;
    // Both rows are split at the same 16-byte boundary.
    if ((reinterpret_cast<uintptr_t>(logits) - reinterpret_cast<uintptr_t>(grad)) % 16 != 0)
      return VCE_EALIGN;
  }
  vce::CeBwdParams p;
  p.logits = logits;
  p.grad = grad;
  p.d1 = d1;
  p.ls0 = ls0;
  p.ls1 = ls1;
  p.V = V;
  p.targets = targets;
  p.ts0 = ts0;
  p.ts1 = ts1;
  p.stats = stats;
  p.n_valid = n_valid;
  p.grad_output = grad_output;
  p.entropy = entropy;
  p.grad_entropy = grad_entropy;
  p.eps = label_smoothing;
  p.reduce_loss = reduce_loss;
  p.ignore_idx = ignore_idx;
  p.v0 = 0;
  p.Vg = V;
  return launch_status(vce::launch_ce_backward(p, dtype, sh.N, static_cast<hipStream_t>(stream)));
}

int ce_forward_backward(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1,
                        int64_t V, int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0,
                        int64_t ts1, const float* grad_output, float label_smoothing,
                        int reduce_loss, int64_t ignore_idx, int overwrite_input,
                        float* loss_tok, float* loss_mean, float* stats, int32_t* n_valid,
                        void* stream) {
  CeShape sh;
  int rc = check_ce_common(logits, dtype, d0, d1, V, ls0, ls1, targets, ts0, ts1,
                           label_smoothing, reduce_loss, &sh);
  if (rc != VCE_OK) return rc;
  if (overwrite_input != 0 && overwrite_input != 1) return VCE_EINVAL;
  if (reduce_loss && (!loss_mean || !n_valid)) return VCE_EINVAL;
  if (sh.N > 0 && (!loss_tok || !stats || !grad || !grad_output)) return VCE_EINVAL;
  if ((stats && !aligned(stats, 16)) || (loss_tok && !aligned(loss_tok, 4)) ||
      (loss_mean && !aligned(loss_mean, 4)) || (n_valid && !aligned(n_valid, 4)) ||
      (grad_output && !aligned(grad_output, 4)))
    return VCE_EALIGN;
  if (sh.N > 0) {
    if (overwrite_input) {
      if (grad != logits) return VCE_EALIAS;
    } else {
      uintptr_t a0, a1, b0, b1;
      extent(logits, d0, d1, V, ls0, ls1, sh.es, &a0, &a1);
      extent(grad, d0, d1, V, ls0, ls1, sh.es, &b0, &b1);
      if (a0 < b1 && b0 < a1) return VCE_EALIAS;
      if ((reinterpret_cast<uintptr_t>(logits) - reinterpret_cast<uintptr_t>(grad)) % 16 != 0)
        return VCE_EALIGN;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  vce::CeMeanParams mp;
  mp.loss_tok = nullptr;
  mp.targets = targets;
  mp.N = sh.N;
  mp.d1 = d1 > 0 ? d1 : 1;
  mp.ts0 = ts0;
  mp.ts1 = ts1;
  mp.ignore_idx = ignore_idx;
  mp.loss_mean = nullptr;
  mp.n_valid = n_valid;
  if (sh.N > 0) {
    // the mean's denominator is needed before the gradient: count first
    if (reduce_loss) {
      rc = launch_status(vce::launch_ce_mean(mp, s));
      if (rc != VCE_OK) return rc;
    }
    vce::CeFwdParams f;
    f.logits = logits;
    f.d1 = d1;
    f.ls0 = ls0;
    f.ls1 = ls1;
    f.V = V;
    f.targets = targets;
    f.ts0 = ts0;
    f.ts1 = ts1;
    f.eps = label_smoothing;
    f.ignore_idx = ignore_idx;
    f.loss_tok = loss_tok;
    f.stats = stats;
    f.entropy = nullptr;
    f.v0 = 0;
    f.partial = nullptr;
    f.partial_w = nullptr;
    vce::CeBwdParams b;
    b.logits = logits;
    b.grad = grad;
    b.d1 = d1;
    b.ls0 = ls0;
    b.ls1 = ls1;
    b.V = V;
    b.targets = targets;
    b.ts0 = ts0;
    b.ts1 = ts1;
    b.stats = stats;
    b.n_valid = n_valid;
    b.grad_output = grad_output;
    b.entropy = nullptr;
    b.grad_entropy = nullptr;
    b.eps = label_smoothing;
    b.reduce_loss = reduce_loss;
    b.ignore_idx = ignore_idx;
    b.v0 = 0;
    b.Vg = V;
    if (vce::ce_fb_fits(dtype, V)) {
      rc = launch_status(vce::launch_ce_forward_backward(f, b, dtype, sh.N, s));
    } else {  // rows too long to hold on chip: the two sweeps
      rc = launch_status(vce::launch_ce_forward(f, dtype, sh.N, s));
      if (rc == VCE_OK) rc = launch_status(vce::launch_ce_backward(b, dtype, sh.N, s));
    }
    if (rc != VCE_OK) return rc;
  }
  if (reduce_loss || n_valid) {
    mp.loss_tok = loss_tok;
    mp.loss_mean = reduce_loss ? loss_mean : nullptr;
    rc = launch_status(vce::launch_ce_mean(mp, s));
  }
  return rc;
}

int ce_forward_shard(const void* logits, int dtype, int64_t d0, int64_t d1, int64_t V_local,
                     int64_t ls0, int64_t ls1, const int64_t* targets, int64_t ts0, int64_t ts1,
                     int64_t vocab_start, int64_t ignore_idx, float* partial, float* partial_w,
                     void* stream) {
  CeShape sh;
  int rc = check_ce_common(logits, dtype, d0, d1, V_local, ls0, ls1, targets, ts0, ts1, 0.0f, 0,
                           &sh);
  if (rc != VCE_OK) return rc;
  if (vocab_start < 0 || vocab_start > INT64_MAX - V_local) return VCE_EINVAL;
  if (sh.N == 0) return VCE_OK;
  if (!partial) return VCE_EINVAL;
  if (!aligned(partial, 16) || (partial_w && !aligned(partial_w, 4))) return VCE_EALIGN;
  vce::CeFwdParams p;
  p.logits = logits;
  p.d1 = d1;
  p.ls0 = ls0;
  p.ls1 = ls1;
  p.V = V_local;
  p.targets = targets;
  p.ts0 = ts0;
  p.ts1 = ts1;
  p.eps = 0.0f;
  p.ignore_idx = ignore_idx;
  p.loss_tok = nullptr;
  p.stats = nullptr;
  p.entropy = nullptr;
  p.v0 = vocab_start;
  p.partial = partial;
  p.partial_w = partial_w;
  return launch_status(vce::launch_ce_forward(p, dtype, sh.N, static_cast<hipStream_t>(stream)));
}

int ce_merge_shards(const float* partials, const float* partials_w, int64_t n_shards, int64_t d0,
                    int64_t d1, const int64_t* targets, int64_t ts0, int64_t ts1, int64_t V,
                    float label_smoothing, int reduce_loss, int64_t ignore_idx, float* loss_tok,
                    float* loss_mean, float* stats, int32_t* n_valid, float* entropy,
                    void* stream) {
  if (n_shards <= 0 || d0 < 0 || d1 < 0 || V <= 0 || ts0 < 0 || ts1 < 0) return VCE_EINVAL;
  if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f)) return VCE_EINVAL;
  if (reduce_loss != 0 && reduce_loss != 1) return VCE_EINVAL;
  int64_t N, tot;
  if (!mul_ok(d0, d1, &N) || N > (int64_t)INT32_MAX) return VCE_EINVAL;
  if (!mul_ok(n_shards, N, &tot) || tot > INT64_MAX / 16) return VCE_EINVAL;
  if (reduce_loss && (!loss_mean || !n_valid)) return VCE_EINVAL;
  if (N > 0 && (!partials || !targets || !loss_tok || !stats)) return VCE_EINVAL;
  if (N > 0 && entropy && !partials_w) return VCE_EINVAL;
  if ((partials_w && !aligned(partials_w, 4)) || (entropy && !aligned(entropy, 4)))
    return VCE_EALIGN;
  if ((partials && !aligned(partials, 16)) || (stats && !aligned(stats, 16)) ||
      (targets && !aligned(targets, 8)) || (loss_tok && !aligned(loss_tok, 4)) ||
      (loss_mean && !aligned(loss_mean, 4)) || (n_valid && !aligned(n_valid, 4)))
    return VCE_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = VCE_OK;
  if (N > 0) {
    vce::CeMergeParams mp;
    mp.partials = partials;
    mp.partials_w = entropy ? partials_w : nullptr;
    mp.entropy = entropy;
    mp.n_shards = n_shards;
    mp.N = N;
    mp.d1 = d1;
    mp.targets = targets;
    mp.ts0 = ts0;
    mp.ts1 = ts1;
    mp.V = V;
    mp.ignore_idx = ignore_idx;
    mp.eps = label_smoothing;
    mp.loss_tok = loss_tok;
    mp.stats = stats;
    rc = launch_status(vce::launch_ce_merge_shards(mp, s));
    if (rc != VCE_OK) return rc;
  }
  if (reduce_loss || n_valid) {
    vce::CeMeanParams mp;
    mp.loss_tok = loss_tok;
    mp.targets = targets;
    mp.N = N;
    mp.d1 = d1 > 0 ? d1 : 1;
    mp.ts0 = ts0;
    mp.ts1 = ts1;
    mp.ignore_idx = ignore_idx;
    mp.loss_mean = reduce_loss ? loss_mean : nullptr;
    mp.n_valid = n_valid;
    rc = launch_status(vce::launch_ce_mean(mp, s));
  }
  return rc;
}

int ce_backward_shard(const void* logits, void* grad, int dtype, int64_t d0, int64_t d1,
                      int64_t V_local, int64_t ls0, int64_t ls1, const int64_t* targets,
                      int64_t ts0, int64_t ts1, int64_t vocab_start, int64_t V,
                      const float* stats, const int32_t* n_valid, const float* grad_output,
                      const float* entropy, const float* grad_entropy, float label_smoothing,
                      int reduce_loss, int64_t ignore_idx, int overwrite_input, void* stream) {
  CeShape sh;
  int rc = check_ce_common(logits, dtype, d0, d1, V_local, ls0, ls1, targets, ts0, ts1,
                           label_smoothing, reduce_loss, &sh);
  if (rc != VCE_OK) return rc;
  if (overwrite_input != 0 && overwrite_input != 1) return VCE_EINVAL;
  if (vocab_start < 0 || V < V_local || vocab_start > V - V_local) return VCE_EINVAL;
  if (sh.N == 0) return VCE_OK;
  if (!grad || !stats || !grad_output || (reduce_loss && !n_valid)) return VCE_EINVAL;
  if (grad_entropy && !entropy) return VCE_EINVAL;
  if (!aligned(stats, 16) || !aligned(grad_output, 4) || (n_valid && !aligned(n_valid, 4)) ||
      (entropy && !aligned(entropy, 4)) || (grad_entropy && !aligned(grad_entropy, 4)))
    return VCE_EALIGN;
  if (overwrite_input) {
    if (grad != logits) return VCE_EALIAS;
  } else {
    uintptr_t a0, a1, b0, b1;
    extent(logits, d0, d1, V_local, ls0, ls1, sh.es, &a0, &a1);
    extent(grad, d0, d1, V_local, ls0, ls1, sh.es, &b0, &b1);
    if (a0 < b1 && b0 < a1) return VCE_EALIAS;
    if ((reinterpret_cast<uintptr_t>(logits) - reinterpret_cast<uintptr_t>(grad)) % 16 != 0)
      return VCE_EALIGN;
  }
  vce::CeBwdParams p;
  p.logits = logits;
  p.grad = grad;
  p.d1 = d1;
  p.ls0 = ls0;
  p.ls1 = ls1;
  p.V = V_local;
  p.targets = targets;
  p.ts0 = ts0;
  p.ts1 = ts1;
  p.stats = stats;
  p.n_valid = n_valid;
  p.grad_output = grad_output;
  p.entropy = grad_entropy ? entropy : nullptr;
  p.grad_entropy = grad_entropy;
  p.eps = label_smoothing;
  p.reduce_loss = reduce_loss;
  p.ignore_idx = ignore_idx;
  p.v0 = vocab_start;
  p.Vg = V;
  return launch_status(vce::launch_ce_backward(p, dtype, sh.N, static_cast<hipStream_t>(stream)));
}

int vce_shift_targets(const int64_t* targets, int64_t d0, int64_t d1, int64_t ts0, int64_t ts1,
                      int seq_axis, int64_t ignore_idx, int64_t* shifted, void* stream) {
  if (d0 < 0 || d1 < 0 || ts0 < 0 || ts1 < 0) return VCE_EINVAL;
  if (seq_axis != 0 && seq_axis != 1) return VCE_EINVAL;
  int64_t N;
  if (!mul_ok(d0, d1, &N)) return VCE_EINVAL;
  if (N == 0) return VCE_OK;
  int64_t span0, span1;
  if (!mul_ok(d0 - 1, ts0, &span0) || !mul_ok(d1 - 1, ts1, &span1) ||
      span0 > INT64_MAX / 8 - span1 - 1)
    return VCE_EINVAL;
  if (!targets || !shifted) return VCE_EINVAL;
  if (!aligned(targets, 8) || !aligned(shifted, 8)) return VCE_EALIGN;
  // the output must not overlap the targets it reads
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(targets);
  const uintptr_t a1 = a0 + (uintptr_t)(span0 + span1 + 1) * 8;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(shifted), b1 = b0 + (uintptr_t)N * 8;
  if (a0 < b1 && b0 < a1) return VCE_EALIAS;
  vce::ShiftParams p;
  p.targets = targets;
  p.d0 = d0;
  p.d1 = d1;
  p.ts0 = ts0;
  p.ts1 = ts1;
  p.N = N;
  p.ignore_idx = ignore_idx;
  p.seq_axis = seq_axis;
  p.out = shifted;
  return launch_status(vce::launch_shift_targets(p, static_cast<hipStream_t>(stream)));
}

size_t lce_workspace_size(int64_t M, int64_t H, int64_t V) {
  vce::LcePlan plan;
  if (!vce::lce_make_plan(M, H, V, &plan)) return 0;
  return plan.total;
}

size_t lce_workspace_size_f32(int64_t M, int64_t H, int64_t V) {
  vce::LcePlan plan;
  if (!vce::lce_make_plan(M, H, V, &plan, true)) return 0;
  return plan.total;
}

namespace {

// static_ws: the forward runs in the library's static scratch (no workspace
// argument; the forward alone must fit in it, VCE_ESCRATCH otherwise).
int check_lce_common(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                     const int64_t* targets, float eps, int reduce_loss, void* workspace,
                     size_t workspace_bytes, vce::LcePlan* plan, bool f32 = false,
                     bool static_ws = false) {
  if (M < 0 || H <= 0 || V <= 0) return VCE_EINVAL;
  if (!(eps >= 0.0f && eps <= 1.0f)) return VCE_EINVAL;
  if (reduce_loss != 0 && reduce_loss != 1) return VCE_EINVAL;
  if (H % 8 != 0) return VCE_EUNSUPPORTED;
  if (!vce::lce_make_plan(M, H, V, plan, f32)) return VCE_EUNSUPPORTED;
  if (static_ws && M > 0 && plan->fwd_bytes > LCE_NOALLOC_SCRATCH_BYTES) return VCE_ESCRATCH;
  if (M == 0) return VCE_OK;
  if (!X || !W || !targets) return VCE_EINVAL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(targets, 8)) return VCE_EALIGN;
  if (static_ws) return VCE_OK;
  if (!workspace) return VCE_EINVAL;
  if (!aligned(workspace, 256)) return VCE_EALIGN;
  if (workspace_bytes < plan->total) return VCE_EWORKSPACE;
  return VCE_OK;
}

// ---- the static scratch of lce_forward_noalloc -------------------------------------
// The forward's per-tile partials for callers that cannot allocate: a file-scope
// device array (each device holds its own copy once the library's code is
// loaded there, until the process ends).  Its name is a host-side stand-in in
// host code; the device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is used.
static __device__ __align__(256) char scratch[LCE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the stream's device (the current device
// for the NULL stream).
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return VCE_EHIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return VCE_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return VCE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return VCE_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return VCE_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return VCE_EHIP;
    if (e != hipSuccess || !p) return VCE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VCE_OK;
}

int lce_forward_impl(bool f32, const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                     const int64_t* targets, float label_smoothing, int reduce_loss,
                     int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                     int32_t* n_valid, float* entropy, void* workspace, size_t workspace_bytes,
                     void* stream, bool static_ws = false, float scale = 1.0f) {
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return VCE_EINVAL;  // finite, positive
  vce::LcePlan plan;
  int rc = check_lce_common(X, W, M, H, V, targets, label_smoothing, reduce_loss, workspace,
                            workspace_bytes, &plan, f32, static_ws);
  if (rc != VCE_OK) return rc;
  if (reduce_loss && (!loss_mean || !n_valid)) return VCE_EINVAL;
  if (M > 0 && (!loss_tok || !stats)) return VCE_EINVAL;
  if (stats && !aligned(stats, 16)) return VCE_EALIGN;
  if ((loss_tok && !aligned(loss_tok, 4)) || (loss_mean && !aligned(loss_mean, 4)) ||
      (n_valid && !aligned(n_valid, 4)) || (entropy && !aligned(entropy, 4)))
    return VCE_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (static_ws && M > 0) {
    rc = scratch_for_stream(s, &workspace);
    if (rc != VCE_OK) return rc;
  }
  if (M > 0) {
    vce::LceFwdArgs a;
    a.X = X;
    a.W = W;
    a.targets = targets;
    a.eps = label_smoothing;
    a.reduce_loss = reduce_loss;
    a.ignore_idx = ignore_idx;
    a.loss_tok = loss_tok;
    a.loss_mean = loss_mean;
    a.stats = stats;
    a.n_valid = n_valid;
    a.entropy = entropy;
    a.ws = static_cast<char*>(workspace);
    a.v0 = 0;
    a.partial = nullptr;
    a.partial_w = nullptr;
    a.scale = scale;
    rc = launch_status(vce::launch_lce_forward(plan, a, s));
    if (rc != VCE_OK) return rc;
  }
  if (reduce_loss || n_valid) {
    vce::CeMeanParams mp;
    mp.loss_tok = loss_tok;
    mp.targets = targets;
    mp.N = M;
    mp.d1 = M > 0 ? M : 1;
    mp.ts0 = 0;
    mp.ts1 = 1;
    mp.ignore_idx = ignore_idx;
    mp.loss_mean = reduce_loss ? loss_mean : nullptr;
    mp.n_valid = n_valid;
    rc = launch_status(vce::launch_ce_mean(mp, s));
  }
  return rc;
}

int lce_backward_impl(bool f32, const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                      const int64_t* targets, const float* stats, const int32_t* n_valid,
                      const float* grad_output, const float* entropy, const float* grad_entropy,
                      float label_smoothing, int reduce_loss, int64_t ignore_idx, void* dX,
                      void* dW, void* workspace, size_t workspace_bytes, void* stream,
                      float scale = 1.0f) {
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return VCE_EINVAL;  // finite, positive
  vce::LcePlan plan;
  int rc = check_lce_common(X, W, M, H, V, targets, label_smoothing, reduce_loss, workspace,
                            workspace_bytes, &plan, f32);
  if (rc != VCE_OK) return rc;
  if (!dW) return VCE_EINVAL;
  if (!aligned(dW, 16)) return VCE_EALIGN;
  if (M > 0) {
    if (!dX || !stats || !grad_output || (reduce_loss && !n_valid)) return VCE_EINVAL;
    if (grad_entropy && !entropy) return VCE_EINVAL;
    if (!aligned(dX, 16) || !aligned(stats, 16) || !aligned(grad_output, 4) ||
        (n_valid && !aligned(n_valid, 4)) || (entropy && !aligned(entropy, 4)) ||
        (grad_entropy && !aligned(grad_entropy, 4)))
      return VCE_EALIGN;
  }
  vce::LceBwdArgs a;
  a.X = X;
  a.W = W;
  a.targets = targets;
  a.stats = stats;
  a.n_valid = n_valid;
  a.grad_output = grad_output;
  a.entropy = grad_entropy ? entropy : nullptr;
  a.grad_entropy = grad_entropy;
  a.eps = label_smoothing;
  a.reduce_loss = reduce_loss;
  a.ignore_idx = ignore_idx;
  a.dX = dX;
  a.dW = dW;
  a.ws = static_cast<char*>(workspace);
  a.v0 = 0;
  a.Vg = V;
  a.scale = scale;
  return launch_status(vce::launch_lce_backward(plan, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int lce_forward(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                const int64_t* targets, float label_smoothing, int reduce_loss,
                int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                int32_t* n_valid, float* entropy, void* workspace, size_t workspace_bytes,
                void* stream) {
  return lce_forward_impl(false, X, W, M, H, V, targets, label_smoothing, reduce_loss,
                          ignore_idx, loss_tok, loss_mean, stats, n_valid, entropy, workspace,
                          workspace_bytes, stream);
}

int lce_forward_scaled(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                       float logit_scale, const int64_t* targets, float label_smoothing,
                       int reduce_loss, int64_t ignore_idx, float* loss_tok, float* loss_mean,
                       float* stats, int32_t* n_valid, float* entropy, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return lce_forward_impl(false, X, W, M, H, V, targets, label_smoothing, reduce_loss,
                          ignore_idx, loss_tok, loss_mean, stats, n_valid, entropy, workspace,
                          workspace_bytes, stream, /*static_ws=*/false, logit_scale);
}

int lce_forward_noalloc(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                        const int64_t* targets, float label_smoothing, int reduce_loss,
                        int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                        int32_t* n_valid, float* entropy, void* stream) {
  return lce_forward_impl(false, X, W, M, H, V, targets, label_smoothing, reduce_loss,
                          ignore_idx, loss_tok, loss_mean, stats, n_valid, entropy, nullptr, 0,
                          stream, /*static_ws=*/true);
}

int lce_forward_f32(const float* X, const float* W, int64_t M, int64_t H, int64_t V,
                    const int64_t* targets, float label_smoothing, int reduce_loss,
                    int64_t ignore_idx, float* loss_tok, float* loss_mean, float* stats,
                    int32_t* n_valid, float* entropy, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return lce_forward_impl(true, X, W, M, H, V, targets, label_smoothing, reduce_loss,
                          ignore_idx, loss_tok, loss_mean, stats, n_valid, entropy, workspace,
                          workspace_bytes, stream);
}

int lce_backward(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                 const int64_t* targets, const float* stats, const int32_t* n_valid,
                 const float* grad_output, const float* entropy, const float* grad_entropy,
                 float label_smoothing, int reduce_loss, int64_t ignore_idx, void* dX, void* dW,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return lce_backward_impl(false, X, W, M, H, V, targets, stats, n_valid, grad_output, entropy,
                           grad_entropy, label_smoothing, reduce_loss, ignore_idx, dX, dW,
                           workspace, workspace_bytes, stream);
}

int lce_backward_scaled(const void* X, const void* W, int64_t M, int64_t H, int64_t V,
                        float logit_scale, const int64_t* targets, const float* stats,
                        const int32_t* n_valid, const float* grad_output, const float* entropy,
                        const float* grad_entropy, float label_smoothing, int reduce_loss,
                        int64_t ignore_idx, void* dX, void* dW, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return lce_backward_impl(false, X, W, M, H, V, targets, stats, n_valid, grad_output, entropy,
                           grad_entropy, label_smoothing, reduce_loss, ignore_idx, dX, dW,
                           workspace, workspace_bytes, stream, logit_scale);
}

int lce_backward_f32(const float* X, const float* W, int64_t M, int64_t H, int64_t V,
                     const int64_t* targets, const float* stats, const int32_t* n_valid,
                     const float* grad_output, const float* entropy, const float* grad_entropy,
                     float label_smoothing, int reduce_loss, int64_t ignore_idx, float* dX,
                     float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  return lce_backward_impl(true, X, W, M, H, V, targets, stats, n_valid, grad_output, entropy,
                           grad_entropy, label_smoothing, reduce_loss, ignore_idx, dX, dW,
                           workspace, workspace_bytes, stream);
}

namespace {

int lce_forward_shard_impl(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                           float scale, const int64_t* targets, int64_t vocab_start,
                           int64_t ignore_idx, float* partial, float* partial_w, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return VCE_EINVAL;  // finite, positive
  vce::LcePlan plan;
  int rc = check_lce_common(X, W, M, H, V_local, targets, 0.0f, 0, workspace, workspace_bytes,
                            &plan);
  if (rc != VCE_OK) return rc;
  if (vocab_start < 0 || vocab_start > INT64_MAX - V_local) return VCE_EINVAL;
  if (M == 0) return VCE_OK;
  if (!partial) return VCE_EINVAL;
  if (!aligned(partial, 16) || (partial_w && !aligned(partial_w, 4))) return VCE_EALIGN;
  vce::LceFwdArgs a;
  a.X = X;
  a.W = W;
  a.targets = targets;
  a.eps = 0.0f;
  a.reduce_loss = 0;
  a.ignore_idx = ignore_idx;
  a.loss_tok = nullptr;
  a.loss_mean = nullptr;
  a.stats = nullptr;
  a.n_valid = nullptr;
  a.entropy = nullptr;
  a.ws = static_cast<char*>(workspace);
  a.v0 = vocab_start;
  a.partial = partial;
  a.partial_w = partial_w;
  a.scale = scale;
  return launch_status(vce::launch_lce_forward(plan, a, static_cast<hipStream_t>(stream)));
}

int lce_backward_shard_impl(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                            float scale, const int64_t* targets, int64_t vocab_start, int64_t V,
                            const float* stats, const int32_t* n_valid, const float* grad_output,
                            const float* entropy, const float* grad_entropy,
                            float label_smoothing, int reduce_loss, int64_t ignore_idx, void* dX,
                            void* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return VCE_EINVAL;  // finite, positive
  vce::LcePlan plan;
  int rc = check_lce_common(X, W, M, H, V_local, targets, label_smoothing, reduce_loss, workspace,
                            workspace_bytes, &plan);
  if (rc != VCE_OK) return rc;
  if (vocab_start < 0 || V < V_local || vocab_start > V - V_local) return VCE_EINVAL;
  if (!dW) return VCE_EINVAL;
  if (!aligned(dW, 16)) return VCE_EALIGN;
  if (M > 0) {
    if (!dX || !stats || !grad_output || (reduce_loss && !n_valid)) return VCE_EINVAL;
    if (grad_entropy && !entropy) return VCE_EINVAL;
    if (!aligned(dX, 16) || !aligned(stats, 16) || !aligned(grad_output, 4) ||
        (n_valid && !aligned(n_valid, 4)) || (entropy && !aligned(entropy, 4)) ||
        (grad_entropy && !aligned(grad_entropy, 4)))
      return VCE_EALIGN;
  }
  vce::LceBwdArgs a;
  a.X = X;
  a.W = W;
  a.targets = targets;
  a.stats = stats;
  a.n_valid = n_valid;
  a.grad_output = grad_output;
  a.entropy = grad_entropy ? entropy : nullptr;
  a.grad_entropy = grad_entropy;
  a.eps = label_smoothing;
  a.reduce_loss = reduce_loss;
  a.ignore_idx = ignore_idx;
  a.dX = dX;
  a.dW = dW;
  a.ws = static_cast<char*>(workspace);
  a.v0 = vocab_start;
  a.Vg = V;
  a.scale = scale;
  return launch_status(vce::launch_lce_backward(plan, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int lce_forward_shard(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                      const int64_t* targets, int64_t vocab_start, int64_t ignore_idx,
                      float* partial, float* partial_w, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return lce_forward_shard_impl(X, W, M, H, V_local, 1.0f, targets, vocab_start, ignore_idx,
                                partial, partial_w, workspace, workspace_bytes, stream);
}

int lce_forward_shard_scaled(const void* X, const void* W, int64_t M, int64_t H,
                             int64_t V_local, float logit_scale, const int64_t* targets,
                             int64_t vocab_start, int64_t ignore_idx, float* partial,
                             float* partial_w, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return lce_forward_shard_impl(X, W, M, H, V_local, logit_scale, targets, vocab_start,
                                ignore_idx, partial, partial_w, workspace, workspace_bytes,
                                stream);
}

int lce_backward_shard(const void* X, const void* W, int64_t M, int64_t H, int64_t V_local,
                       const int64_t* targets, int64_t vocab_start, int64_t V,
                       const float* stats, const int32_t* n_valid, const float* grad_output,
                       const float* entropy, const float* grad_entropy, float label_smoothing,
                       int reduce_loss, int64_t ignore_idx, void* dX, void* dW, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return lce_backward_shard_impl(X, W, M, H, V_local, 1.0f, targets, vocab_start, V, stats,
                                 n_valid, grad_output, entropy, grad_entropy, label_smoothing,
                                 reduce_loss, ignore_idx, dX, dW, workspace, workspace_bytes,
                                 stream);
}

int lce_backward_shard_scaled(const void* X, const void* W, int64_t M, int64_t H,
                              int64_t V_local, float logit_scale, const int64_t* targets,
                              int64_t vocab_start, int64_t V, const float* stats,
                              const int32_t* n_valid, const float* grad_output,
                              const float* entropy, const float* grad_entropy,
                              float label_smoothing, int reduce_loss, int64_t ignore_idx,
                              void* dX, void* dW, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return lce_backward_shard_impl(X, W, M, H, V_local, logit_scale, targets, vocab_start, V,
                                 stats, n_valid, grad_output, entropy, grad_entropy,
                                 label_smoothing, reduce_loss, ignore_idx, dX, dW, workspace,
                                 workspace_bytes, stream);
}

int vce_gemm_bf16(const void* P, int64_t ldp, int p_dim, const void* Q, int64_t ldq, int q_dim,
                  int64_t rows, int64_t cols, int64_t K, float* C, int64_t ldc, void* stream) {
  if (rows < 0 || cols < 0 || K < 0) return VCE_EINVAL;
  if ((p_dim != 0 && p_dim != 1) || (q_dim != 0 && q_dim != 1)) return VCE_EINVAL;
  if (rows == 0 || cols == 0) return VCE_OK;
  if (!P || !Q || !C) return VCE_EINVAL;
  // the contiguous axis is masked per 8-element chunk
  if (!p_dim && K % 8 != 0) return VCE_EUNSUPPORTED;
  if (!q_dim && K % 8 != 0) return VCE_EUNSUPPORTED;
  if (p_dim && rows % 8 != 0) return VCE_EUNSUPPORTED;
  if (q_dim && cols % 8 != 0) return VCE_EUNSUPPORTED;
  if (ldp % 8 != 0 || ldq % 8 != 0) return VCE_EUNSUPPORTED;
  if (ldc < cols || ldp < (p_dim ? rows : K) || ldq < (q_dim ? cols : K)) return VCE_EINVAL;
  // 256 rows x leading dimension x 2 bytes must stay below 2^31 (buffer offsets)
  if (ldp > ((int64_t)1 << 22) || ldq > ((int64_t)1 << 22)) return VCE_EUNSUPPORTED;
  if (rows > ((int64_t)1 << 31) || cols > ((int64_t)1 << 31)) return VCE_EUNSUPPORTED;
  if (!aligned(P, 16) || !aligned(Q, 16) || !aligned(C, 4)) return VCE_EALIGN;
  return launch_status(vce::launch_gemm_bf16(P, ldp, p_dim, Q, ldq, q_dim, rows, cols, K, C, ldc,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
