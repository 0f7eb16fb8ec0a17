// Kernel parameter blocks and launchers shared by the C-ABI layer and the
// kernel translation units of libvce.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vce {

struct CeFwdParams {
  const void* logits;
  int64_t d1, ls0, ls1, V;
  const int64_t* targets;
  int64_t ts0, ts1;
  float eps;
  int64_t ignore_idx;
  float* loss_tok;
  float* stats;
  float* entropy;  // optional (N)
  int64_t v0;      // first vocabulary column of the row (0 unless sharded)
  float* partial;  // shard mode: (N, 4) partial statistics instead of loss/stats
  float* partial_w;  // shard mode, optional: (N) entropy statistic w of the shard
};

struct CeMergeParams {
  const float* partials;    // (n_shards, N, 4)
  const float* partials_w;  // with entropy: (n_shards, N)
  int64_t n_shards, N, d1;
  const int64_t* targets;
  int64_t ts0, ts1, V, ignore_idx;  // V: the full vocabulary
  float eps;
  float* loss_tok;
  float* stats;
  float* entropy;  // optional (N), needs partials_w
};

struct CeMeanParams {
  const float* loss_tok;
  const int64_t* targets;
  int64_t N, d1, ts0, ts1, ignore_idx;
  float* loss_mean;
  int32_t* n_valid;
};

struct CeBwdParams {
  const void* logits;
  void* grad;
  int64_t d1, ls0, ls1, V;
  const int64_t* targets;
  int64_t ts0, ts1;
  const float* stats;
  const int32_t* n_valid;
  const float* grad_output;
  const float* entropy;       // with grad_entropy: the forward's entropy (N)
  const float* grad_entropy;  // optional (N): adds grad_entropy[r] dH/dz
  float eps;
  int reduce_loss;
  int64_t ignore_idx;
  int64_t v0, Vg;  // the row holds columns v0 .. v0 + V - 1 of Vg (0, V unless sharded)
  int splits = 1;  // workgroups per row (set by the launcher)
};

hipError_t launch_ce_forward(const CeFwdParams& p, int dtype, int64_t N, hipStream_t stream);
hipError_t launch_ce_mean(const CeMeanParams& p, hipStream_t stream);
hipError_t launch_ce_merge_shards(const CeMergeParams& p, hipStream_t stream);

struct ShiftParams {
  const int64_t* targets;
  int64_t d0, d1, ts0, ts1, N, ignore_idx;
  int seq_axis;
  int64_t* out;
};
hipError_t launch_shift_targets(const ShiftParams& p, hipStream_t stream);
hipError_t launch_ce_backward(const CeBwdParams& p, int dtype, int64_t N, hipStream_t stream);
// One-pass forward + backward (rows of at most 512 x 32 16-byte vectors: see ce_fb_fits).
bool ce_fb_fits(int dtype, int64_t V);
hipError_t launch_ce_forward_backward(const CeFwdParams& f, const CeBwdParams& b, int dtype,
                                      int64_t N, hipStream_t stream);

// ---- fused linear cross-entropy ----------------------------------------------

// Workspace plan of the linear form for an (M, H, V) problem.
struct LcePlan {
  int64_t M, H, V;
  int64_t Mp;          // M rounded up to the token tile
  int64_t n_vtiles;    // vocabulary tiles of the forward
  int64_t chunk;       // vocabulary rows per backward chunk (multiple of the tile)
  int64_t n_chunks;
  int64_t ldz;         // row stride (elements) of the dZ chunk buffer
  size_t off_part;     // forward: per-tile partials and target logits
  size_t off_dz, off_dx;  // backward: dZ of one chunk, FP32 dX accumulator
  size_t off_dz2;         // second dZ buffer (BF16 form, several chunks), else off_dz
  size_t fwd_bytes;       // what the forward alone uses (from offset 0)
  size_t total;
  // FP32 inputs: X and W split into BF16 hi and lo planes in the workspace
  // (lo plane right after its hi plane), dZ in two planes, no accumulator
  // (dX is FP32 and accumulates in place)
  bool f32;
  size_t off_xs, off_ws;  // hi planes of X and W
  size_t xplane, wplane;  // bytes per plane
  int64_t dzplane;        // elements from the hi plane of dZ to its lo plane
};

bool lce_make_plan(int64_t M, int64_t H, int64_t V, LcePlan* plan, bool f32 = false);

struct LceFwdArgs {
  const void* X;
  const void* W;
  const int64_t* targets;
  float eps;
  int reduce_loss;
  int64_t ignore_idx;
  float* loss_tok;
  float* loss_mean;
  float* stats;
  int32_t* n_valid;
  float* entropy;  // optional (M)
  char* ws;
  int64_t v0;      // vocabulary index of W's first row (0 unless sharded)
  float* partial;  // shard mode: (M, 4) local statistics instead of loss/stats
  float* partial_w;  // shard mode, optional: (M) entropy statistic w of the shard
  float scale = 1.0f;  // logits = scale X W^T (scale > 0)
};

struct LceBwdArgs {
  const void* X;
  const void* W;
  const int64_t* targets;
  const float* stats;
  const int32_t* n_valid;
  const float* grad_output;
  const float* entropy;       // with grad_entropy: the forward's entropy (M)
  const float* grad_entropy;  // optional (M)
  float eps;
  int reduce_loss;
  int64_t ignore_idx;
  void* dX;
  void* dW;
  char* ws;
  int64_t v0, Vg;  // W holds vocabulary rows v0 .. v0 + V - 1 of Vg (0, V unless sharded)
  float scale = 1.0f;  // logits = scale X W^T (scale > 0)
};

hipError_t launch_lce_forward(const LcePlan& plan, const LceFwdArgs& a, hipStream_t stream);
hipError_t launch_lce_backward(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream);
hipError_t launch_gemm_bf16(const void* P, int64_t ldp, int p_dim, const void* Q, int64_t ldq,
                            int q_dim, int64_t rows, int64_t cols, int64_t K, float* C,
                            int64_t ldc, hipStream_t stream);

}  // namespace vce
