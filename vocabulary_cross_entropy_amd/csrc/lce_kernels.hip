// Fused linear cross-entropy for gfx950: logits = X W^T are produced tile by
// tile on the matrix cores and consumed in the GEMM epilogue, never stored.
//
// What is computed follows the cut-cross-entropy package description (loss
// of linear_cross_entropy from embeddings, classifier and labels: target
// logit and log-sum-exp over the whole vocabulary, logits kept on chip) and
// the Liger-Kernel fused linear cross-entropy PR (Summary: classifier GEMM
// fused with NLL/LSE; Backward: dZ from recomputed logits, then dX and dW;
// Performance methodology: four GEMMs for forward+backward).
//
// Design for CDNA4 (not the SM100 design of that PR):
//  * One GEMM core: a 256 x 256 output tile per 256-thread workgroup, four
//    wavefronts of 128 x 128, v_mfma_f32_32x32x16_bf16, K staged through LDS
//    in 64-deep slices, double buffered (128 KB of the 160 KB LDS), one
//    barrier per slice.  16-byte chunks are XOR-swizzled across rows so the
//    fragment reads and the tile writes avoid bank conflicts.  An operand may
//    be stored K-contiguous or dim-contiguous; the latter is transposed in
//    registers (8 x 8 BF16 blocks) on its way into LDS, so every GEMM of the
//    backward reads X, W and dZ in place.
//  * Forward: tiles are (vocabulary x tokens); each lane owns tokens, so the
//    epilogue reduces the online LSE (max, sum of exp, sum of logits) over the
//    vocabulary inside the lane, then across the two lane halves and the two
//    wavefronts that share the tokens.  Per-tile partials are merged per
//    token by a second kernel in a fixed order.
//  * Backward: the vocabulary is processed in chunks.  Per chunk: recompute
//    the logits and write dZ (BF16) to the workspace; dW rows of the chunk are
//    finished by one GEMM over all tokens (written once, never accumulated);
//    dX accumulates chunk by chunk in an FP32 buffer, the last chunk writes
//    BF16.
//  * Tile order is XCD-aware: consecutive workgroups go round-robin over the
//    8 XCDs, so each XCD is given a contiguous range of tiles, in which
//    neighbouring tiles share their vocabulary slice of W (L2 reuse).
#include "vce_device.h"
#include "vce_internal.h"

namespace vce {

namespace {

constexpr int BM = 256;   // output rows per tile (P side)
constexpr int BN = 256;   // output cols per tile (Q side)
constexpr int BK = 64;    // K slice
constexpr int NT = 256;   // threads per workgroup
constexpr int kLdsElems = 2 * (BM + BN) * BK;  // two stages of P and Q, BF16
constexpr int64_t kChunk = 32768;              // backward vocabulary chunk

static_assert(BM == BN, "the tile loaders assume square tiles");

// An operand of C[i][j] = sum_k P(i, k) Q(j, k).
//   K-contiguous:   element (d, k) at base[d * ld + k]
//   dim-contiguous: element (d, k) at base[k * ld + d]
// dim_limit: d >= dim_limit reads as 0.  k_limit: k >= k_limit reads as 0.
// For K-contiguous operands k is tested per 8-element chunk (chunk start),
// for dim-contiguous ones d is tested per 8-element chunk.
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int64_t dim_limit;
  int64_t k_limit;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row ^ (row >> 3)) & 7);
}

template <bool KC>
struct TileLoader;

// K-contiguous: 256 rows x 8 chunks; thread t loads chunk (t & 7) of rows
// (t >> 3) + 32 i: eight threads cover one row's 128 contiguous bytes.
template <>
struct TileLoader<true> {
  u32x4_t r[8];
  __device__ __forceinline__ void load(const Operand& op, int64_t d0, int64_t k0, int tid) {
    const int c = tid & 7;
    const int64_t k = k0 + c * 8;
    const bool kok = k < op.k_limit;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t d = d0 + (tid >> 3) + 32 * i;
      if (kok && d < op.dim_limit)
        r[i] = *reinterpret_cast<const u32x4_t*>(op.base + d * op.ld + k);
      else
        r[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4_t*>(s + row * BK + swz(row, c) * 8) = r[i];
    }
  }
};

// dim-contiguous: 64 k-rows x 256 dims; thread t loads the 8 x 8 block of
// k-rows 8 (t >> 5) .. +7 and dims 8 (t & 31) .. +7 (32 threads cover 512
// contiguous bytes of one k-row), then transposes it so LDS holds dim-rows.
template <>
struct TileLoader<false> {
  u32x4_t r[8];
  __device__ __forceinline__ void load(const Operand& op, int64_t d0, int64_t k0, int tid) {
    const int kb = tid >> 5, db = tid & 31;
    const int64_t d = d0 + db * 8;
    const bool dok = d < op.dim_limit;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int64_t k = k0 + kb * 8 + kk;
      if (dok && k < op.k_limit)
        r[kk] = *reinterpret_cast<const u32x4_t*>(op.base + k * op.ld + d);
      else
        r[kk] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
    const int kb = tid >> 5, db = tid & 31;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int q = dd >> 1;
      u32x4_t o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = r[2 * p][q], hi = r[2 * p + 1][q];
        o[p] = (dd & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int row = db * 8 + dd;
      *reinterpret_cast<u32x4_t*>(s + row * BK + swz(row, kb) * 8) = o;
    }
  }
};

__device__ __forceinline__ bf16x8_t frag(const uint16_t* s, int row, int chunk) {
  return __builtin_bit_cast(bf16x8_t,
                            *reinterpret_cast<const u32x4_t*>(s + row * BK + swz(row, chunk) * 8));
}

// Hardware workgroup id -> logical tile: the dispatcher deals workgroups to
// the 8 XCDs round-robin; give XCD x the contiguous logical range
// [x q + min(x, rem), ...) so neighbouring tiles run on the same L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n >> 3, rem = n & 7;
  const int x = b & 7, slot = b >> 3;
  return x * q + (x < rem ? x : rem) + slot;
}

// Output element of accumulator register r of block (a, b) for this lane:
//   row i = i0 + 128 wr + 32 a + 8 (r / 4) + 4 (lane / 32) + r % 4
//   col j = j0 + 128 wc + 32 b + lane % 32
template <bool PKC, bool QKC, class Epi>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(Operand P, Operand Q, int64_t K, int n_tj,
                                                   int n_tiles, typename Epi::Params ep) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kLdsElems];
  // stage s: P slice at smem + s * BM * BK, Q slice at smem + 2 * BM * BK + s * BN * BK
  uint16_t* const sQbase = smem + 2 * BM * BK;

  const int tile = xcd_remap(blockIdx.x, n_tiles);
  const int ti = tile / n_tj, tj = tile - (tile / n_tj) * n_tj;
  const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  TileLoader<PKC> lp;
  TileLoader<QKC> lq;
  const int nk = (int)((K + BK - 1) / BK);
  lp.load(P, i0, 0, tid);
  lq.load(Q, j0, 0, tid);
  lp.store(smem, tid);
  lq.store(sQbase, tid);
  __syncthreads();

  const int prow = wr * 128 + (lane & 31), qrow = wc * 128 + (lane & 31);
  const int khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      lp.load(P, i0, (int64_t)(kt + 1) * BK, tid);
      lq.load(Q, j0, (int64_t)(kt + 1) * BK, tid);
    }
    const uint16_t* cp = smem + cur * (BM * BK);
    const uint16_t* cq = sQbase + cur * (BN * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) fa[a] = frag(cp, prow + 32 * a, 2 * ks + khalf);
#pragma unroll
      for (int b = 0; b < 4; ++b) fb[b] = frag(cq, qrow + 32 * b, 2 * ks + khalf);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      lp.store(smem + (cur ^ 1) * (BM * BK), tid);
      lq.store(sQbase + (cur ^ 1) * (BN * BK), tid);
    }
    __syncthreads();
  }
  Epi::apply(ep, acc, i0, j0, wr, wc, lane, smem);
}

// ---- epilogues ------------------------------------------------------------------

// Plain FP32 store (the exported building block).
struct EpiF32 {
  struct Params {
    float* C;
    int64_t ldc, rows, cols;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][4], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + wc * 128 + b * 32 + (lane & 31);
      if (j >= p.cols) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = i0 + wr * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (i < p.rows) p.C[i * p.ldc + j] = acc[a][b][r];
        }
    }
  }
};

// Forward: rows = vocabulary, cols = tokens.  Per token and vocabulary tile:
// (max, sum exp(z - max), sum z) into the partial arrays, plus the target
// logit written by the one lane that holds it.
struct EpiLse {
  struct Params {
    float* pm;
    float* pd;
    float* ps;
    float* zt;
    const int64_t* targets;
    int64_t M, V, Mp, ignore_idx;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][4], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t* smem) {
    float* sh = reinterpret_cast<float*>(smem);  // [wr][wc][b][lane 0..31][3]
    const int64_t vbase = i0 + wr * 128 + 4 * (lane >> 5);
    // rows at offsets >= lim from vbase lie beyond the vocabulary
    const int64_t lim64 = p.V - vbase;
    const int lim = lim64 > 128 ? 128 : (lim64 < 0 ? 0 : (int)lim64);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + wc * 128 + b * 32 + (lane & 31);
      float mx = kNegInf;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (a * 32 + 8 * (r >> 2) + (r & 3) < lim) mx = fmaxf(mx, acc[a][b][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mref = (mx == kNegInf) ? 0.0f : mx;
      const float mL = mref * kLog2e;
      float d = 0.0f, s = 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (a * 32 + 8 * (r >> 2) + (r & 3) < lim) {
            d += exp2_hw(__builtin_fmaf(acc[a][b][r], kLog2e, -mL));
            s += acc[a][b][r];
          }
      d += __shfl_xor(d, 32, 64);
      s += __shfl_xor(s, 32, 64);
      // Target logit: the lane holding row t picks it with a two-level select
      // (row block a, then register r), no dynamic register index.
      if (j < p.M) {
        const int64_t t = p.targets[j];
        const int64_t tl64 = t - vbase;
        const bool inr = t != p.ignore_idx && tl64 >= 0 && tl64 < 128 && ((tl64 >> 2) & 1) == 0;
        const int tl = inr ? (int)tl64 : 0;
        const int ra = tl >> 5, rr = ((tl >> 3) & 3) * 4 + (tl & 3);
        float zt = 0.0f;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float x = acc[a][b][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) x = (rr == r) ? acc[a][b][r] : x;
          zt = (ra == a) ? x : zt;
        }
        if (inr) p.zt[j] = zt;
      }
      if (lane < 32) {
        float* e = sh + (((wr * 2 + wc) * 4 + b) * 32 + lane) * 3;
        e[0] = mx;
        e[1] = d;
        e[2] = s;
      }
    }
    __syncthreads();
    // one wavefront per token column half merges the two vocabulary halves
    if (wr == 0 && lane < 32) {
      const int64_t vt = i0 / BM;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t j = j0 + wc * 128 + b * 32 + lane;
        const float* e0 = sh + (((0 * 2 + wc) * 4 + b) * 32 + lane) * 3;
        const float* e1 = sh + (((1 * 2 + wc) * 4 + b) * 32 + lane) * 3;
        LseState st{e0[0], e0[1], e0[2]};
        lse_merge(st, LseState{e1[0], e1[1], e1[2]});
        if (j < p.M) {
          p.pm[vt * p.Mp + j] = st.m;
          p.pd[vt * p.Mp + j] = st.d;
          p.ps[vt * p.Mp + j] = st.s;
        }
      }
    }
  }
};

// Backward dZ: rows = vocabulary of the chunk, cols = tokens.
// dZ = g (exp(z - lse) - (1-eps)[v = t] - eps/V), stored BF16 token-major.
struct EpiDz {
  struct Params {
    uint16_t* dz;
    int64_t ldz, c0, vc_valid;
    const float* stats;
    const int64_t* targets;
    const float* grad_output;
    const int32_t* n_valid;
    float eps;
    int reduce_loss;
    int64_t ignore_idx, M, V;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][4], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
    float gscale = 0.0f;
    if (p.reduce_loss) {
      const int32_t nv = p.n_valid[0];
      gscale = p.grad_output[0] / (float)(nv > 0 ? nv : 1);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + wc * 128 + b * 32 + (lane & 31);
      int64_t t = -1;
      float g = 0.0f, lse2 = 0.0f;
      bool live = false, bad = false;
      if (j < p.M) {
        t = p.targets[j];
        if (t != p.ignore_idx) {
          if (t >= 0 && t < p.V) {
            live = true;
            g = p.reduce_loss ? gscale : p.grad_output[j];
            const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(p.stats + 4 * j);
            lse2 = sv[0] * kLog2e + log2_hw(sv[1]);
          } else {
            bad = true;
          }
        }
      }
      const float goff = g * (p.eps / (float)p.V);
      const float gt = g * (1.0f - p.eps);
      // Offsets relative to this lane's first row keep the per-element tests
      // in 32-bit compares against constants.
      const int64_t vrow0 = i0 + wr * 128 + 4 * (lane >> 5);  // chunk-local row of r = 0
      const int64_t tr64 = t - p.c0 - vrow0;
      const int trel = (live && tr64 >= 0 && tr64 < 128) ? (int)tr64 : -1;
      const int64_t lim64 = p.vc_valid - vrow0;
      const int lim = lim64 > 128 ? 128 : (lim64 < 0 ? 0 : (int)lim64);
      const float fill = bad ? __builtin_nanf("") : 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float val[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int off = a * 32 + 8 * q + e;
            float x = g * exp2_hw(__builtin_fmaf(acc[a][b][4 * q + e], kLog2e, -lse2)) - goff;
            x = (off == trel) ? x - gt : x;
            val[e] = (live && off < lim) ? x : fill;
          }
          u32x2_t w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
          *reinterpret_cast<u32x2_t*>(p.dz + j * p.ldz + vrow0 + a * 32 + 8 * q) = w;
        }
    }
  }
};

// Backward dW of a chunk: rows = hidden (h), cols = vocabulary of the chunk.
struct EpiDw {
  struct Params {
    uint16_t* dW;
    int64_t H, c0, vc_valid;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][4], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + wc * 128 + b * 32 + (lane & 31);
      if (j >= p.vc_valid) continue;
      uint16_t* row = p.dW + (p.c0 + j) * p.H;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t i = i0 + wr * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
          if (i < p.H) {
            u32x2_t w = {pack_bf16x2(acc[a][b][4 * q], acc[a][b][4 * q + 1]),
                         pack_bf16x2(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3])};
            *reinterpret_cast<u32x2_t*>(row + i) = w;
          }
        }
    }
  }
};

// Backward dX: rows = hidden (h), cols = tokens.  mode bit 0: add the FP32
// accumulator of earlier chunks; bit 1: final chunk, write BF16 dX.
struct EpiDx {
  struct Params {
    float* accbuf;
    uint16_t* dX;
    int64_t H, M;
    int mode;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][4], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + wc * 128 + b * 32 + (lane & 31);
      if (j >= p.M) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t i = i0 + wr * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
          if (i >= p.H) continue;
          f32x4_t v = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                       acc[a][b][4 * q + 3]};
          float* ap = p.accbuf + j * p.H + i;
          if (p.mode & 1) v += *reinterpret_cast<const f32x4_t*>(ap);
          if (p.mode & 2) {
            u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2_t*>(p.dX + j * p.H + i) = w;
          } else {
            *reinterpret_cast<f32x4_t*>(ap) = v;
          }
        }
    }
  }
};

// Per-token merge of the forward partials (fixed order), then loss and stats.
struct MergeParams {
  const float* pm;
  const float* pd;
  const float* ps;
  const float* zt;
  const int64_t* targets;
  int64_t M, Mp, V, n_vt, ignore_idx;
  float eps;
  float* loss_tok;
  float* stats;
};

__global__ __launch_bounds__(256) void lce_merge_kernel(MergeParams p) {
  __shared__ LseState sh[8][32];
  const int tl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + tl;
  LseState st = {kNegInf, 0.0f, 0.0f};
  if (j < p.M) {
    for (int64_t vt = grp; vt < p.n_vt; vt += 8) {
      const int64_t o = vt * p.Mp + j;
      lse_merge(st, LseState{p.pm[o], p.pd[o], p.ps[o]});
    }
  }
  sh[grp][tl] = st;
  __syncthreads();
  if (grp != 0 || j >= p.M) return;
  for (int g = 1; g < 8; ++g) lse_merge(st, sh[g][tl]);
  const int64_t t = p.targets[j];
  if (t == p.ignore_idx) {
    p.loss_tok[j] = 0.0f;
    *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    return;
  }
  const bool t_ok = t >= 0 && t < p.V;
  const float zt = t_ok ? p.zt[j] : __builtin_nanf("");
  const float mean = st.s / (float)p.V;
  float loss = log2_hw(st.d) * kLn2 - (1.0f - p.eps) * (zt - st.m);
  if (p.eps != 0.0f) loss -= p.eps * (mean - st.m);
  p.loss_tok[j] = t_ok ? loss : __builtin_nanf("");
  *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{st.m, st.d, zt, mean};
}

template <bool PKC, bool QKC, class Epi>
hipError_t run_gemm(const Operand& P, const Operand& Q, int64_t rows, int64_t cols, int64_t K,
                    const typename Epi::Params& ep, hipStream_t stream) {
  const int64_t n_ti = (rows + BM - 1) / BM, n_tj = (cols + BN - 1) / BN;
  const int64_t n = n_ti * n_tj;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<PKC, QKC, Epi>), dim3((unsigned)n), dim3(NT), 0, stream, P, Q,
                     K, (int)n_tj, (int)n, ep);
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool lce_make_plan(int64_t M, int64_t H, int64_t V, LcePlan* plan) {
  if (M < 0 || H <= 0 || V <= 0 || H % 8 != 0) return false;
  if (M > ((int64_t)1 << 31) || V > ((int64_t)1 << 31) || H > ((int64_t)1 << 20)) return false;
  LcePlan p;
  p.M = M;
  p.H = H;
  p.V = V;
  p.Mp = ((M > 0 ? M : 1) + BN - 1) / BN * BN;
  p.n_vtiles = (V + BM - 1) / BM;
  const int64_t vr = (V + BM - 1) / BM * BM;
  p.chunk = vr < kChunk ? vr : kChunk;
  p.n_chunks = (V + p.chunk - 1) / p.chunk;
  p.ldz = p.chunk;
  const size_t part = align256((size_t)p.n_vtiles * p.Mp * 4);
  p.off_part = 0;
  const size_t fwd = 3 * part + align256((size_t)p.Mp * 4);
  const size_t dz = align256((size_t)p.Mp * p.ldz * 2);
  const size_t dx = p.n_chunks > 1 ? align256((size_t)p.Mp * H * 4) : 0;
  p.off_dz = 0;
  p.off_dx = dz;
  p.total = fwd > dz + dx ? fwd : dz + dx;
  *plan = p;
  return true;
}

hipError_t launch_lce_forward(const LcePlan& plan, const LceFwdArgs& a, hipStream_t stream) {
  const size_t part = align256((size_t)plan.n_vtiles * plan.Mp * 4);
  float* pm = reinterpret_cast<float*>(a.ws + plan.off_part);
  float* pd = reinterpret_cast<float*>(a.ws + plan.off_part + part);
  float* ps = reinterpret_cast<float*>(a.ws + plan.off_part + 2 * part);
  float* zt = reinterpret_cast<float*>(a.ws + plan.off_part + 3 * part);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  Operand P{W, plan.H, plan.V, plan.H};
  Operand Q{X, plan.H, plan.M, plan.H};
  EpiLse::Params ep{pm, pd, ps, zt, a.targets, plan.M, plan.V, plan.Mp, a.ignore_idx};
  hipError_t e = run_gemm<true, true, EpiLse>(P, Q, plan.V, plan.Mp, plan.H, ep, stream);
  if (e != hipSuccess) return e;
  MergeParams mp{pm, pd, ps, zt, a.targets, plan.M, plan.Mp, plan.V, plan.n_vtiles,
                 a.ignore_idx, a.eps, a.loss_tok, a.stats};
  hipLaunchKernelGGL(lce_merge_kernel, dim3((unsigned)((plan.M + 31) / 32)), dim3(256), 0, stream,
                     mp);
  return hipGetLastError();
}

hipError_t launch_lce_backward(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream) {
  if (plan.M == 0) return hipSuccess;  // dW of an empty batch: nothing reads it
  uint16_t* dz = reinterpret_cast<uint16_t*>(a.ws + plan.off_dz);
  float* dxacc = reinterpret_cast<float*>(a.ws + plan.off_dx);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  for (int64_t c = 0; c < plan.n_chunks; ++c) {
    const int64_t c0 = c * plan.chunk;
    const int64_t vc = (plan.V - c0) < plan.chunk ? (plan.V - c0) : plan.chunk;
    const uint16_t* Wc = W + c0 * plan.H;
    // dZ of the chunk: (vocabulary x tokens), K = H
    {
      Operand P{Wc, plan.H, vc, plan.H};
      Operand Q{X, plan.H, plan.M, plan.H};
      EpiDz::Params ep{dz, plan.ldz, c0, vc, a.stats, a.targets, a.grad_output, a.n_valid,
                       a.eps, a.reduce_loss, a.ignore_idx, plan.M, plan.V};
      hipError_t e = run_gemm<true, true, EpiDz>(P, Q, vc, plan.Mp, plan.H, ep, stream);
      if (e != hipSuccess) return e;
    }
    // dW rows of the chunk: (hidden x vocabulary), K = tokens
    {
      Operand P{X, plan.H, plan.H, plan.M};
      Operand Q{dz, plan.ldz, plan.ldz, plan.M};
      EpiDw::Params ep{static_cast<uint16_t*>(a.dW), plan.H, c0, vc};
      hipError_t e = run_gemm<false, false, EpiDw>(P, Q, plan.H, vc, plan.M, ep, stream);
      if (e != hipSuccess) return e;
    }
    // dX += dZ_c W_c: (hidden x tokens), K = vocabulary of the chunk
    {
      Operand P{Wc, plan.H, plan.H, vc};
      Operand Q{dz, plan.ldz, plan.M, (vc + 7) / 8 * 8};
      const int mode = (c > 0 ? 1 : 0) | (c + 1 == plan.n_chunks ? 2 : 0);
      EpiDx::Params ep{dxacc, static_cast<uint16_t*>(a.dX), plan.H, plan.M, mode};
      hipError_t e = run_gemm<false, true, EpiDx>(P, Q, plan.H, plan.M, vc, ep, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const void* P, int p_kmajor, int64_t ldp, const void* Q, int q_kmajor,
                            int64_t ldq, int64_t rows, int64_t cols, int64_t K, float* C,
                            int64_t ldc, hipStream_t stream) {
  Operand op{static_cast<const uint16_t*>(P), ldp, rows, K};
  Operand oq{static_cast<const uint16_t*>(Q), ldq, cols, K};
  EpiF32::Params ep{C, ldc, rows, cols};
  if (p_kmajor && q_kmajor) return run_gemm<true, true, EpiF32>(op, oq, rows, cols, K, ep, stream);
  if (p_kmajor) return run_gemm<true, false, EpiF32>(op, oq, rows, cols, K, ep, stream);
  if (q_kmajor) return run_gemm<false, true, EpiF32>(op, oq, rows, cols, K, ep, stream);
  return run_gemm<false, false, EpiF32>(op, oq, rows, cols, K, ep, stream);
}

}  // namespace vce
