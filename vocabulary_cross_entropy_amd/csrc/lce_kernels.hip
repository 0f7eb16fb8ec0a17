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
//  * One GEMM core, C[i][j] = sum_k P[i][k] Q[j][k] with both operands stored
//    K-contiguous: a 256 x 256 output tile per 512-thread workgroup, eight
//    wavefronts (two per SIMD, so one wave's waits overlap the other's
//    matrix work) of 128 x 64 each, v_mfma_f32_32x32x16_bf16.  K advances in
//    64-deep slices through two LDS stages (128 KB of the 160 KB); global
//    data goes straight to LDS (buffer_load ... lds).  The two wavefronts of
//    each SIMD run ping-pong: while one issues its fragment reads and loads,
//    the other runs 16 MFMAs back to back (measured on MI355X: 13% fewer
//    cycles per slice than interleaving both kinds in every wave).  16-byte chunks are XOR-swizzled across rows (the loads
//    pick their source addresses so the linear LDS writes land swizzled) and
//    the fragment reads are bank-conflict free.
//  * Tile order: hardware workgroup ids go round-robin over the 8 XCDs, so
//    each XCD is given a contiguous range of tiles, walked in bands of 8 row
//    tiles so the 32 workgroups an XCD runs at once share both operands in
//    its L2.
//  * Forward: tiles are (vocabulary x tokens); each lane owns tokens, so the
//    epilogue reduces the online LSE (max, sum of exp, sum of logits) over the
//    vocabulary inside the lane, then across the two lane halves and the two
//    wavefronts that share the tokens.  Per-tile partials are merged per
//    token by a second kernel in a fixed order.
//  * Backward, per vocabulary chunk: recompute the logits and write dZ (BF16)
//    token-major and vocabulary-major; dW rows of the chunk are finished by
//    one GEMM over all tokens (written once, never accumulated); dX
//    accumulates chunk by chunk in FP32, the last chunk writes BF16.  The
//    K-contiguous copies this needs (X^T once per call, W_c^T per chunk) are
//    made by an LDS-tiled transpose; they cost a few percent of the GEMM time.
#include "vce_device.h"
#include "vce_internal.h"

namespace vce {

namespace {

constexpr int BM = 256;   // output rows per tile (P side)
constexpr int BN = 256;   // output cols per tile (Q side)
constexpr int BK = 64;    // K slice per stage
constexpr int NT = 512;   // threads per workgroup: 8 wavefronts
constexpr int WN = 64;    // output cols per wavefront
constexpr int NB = WN / 32;                        // 32-column blocks per wavefront
constexpr int ROWS_PER_LD = 1024 / (BK * 2);       // rows one 1 KB LDS load covers (8)
constexpr int LD_PER_WAVE = BM / 8 / ROWS_PER_LD;  // loads per wave per operand per slice (4)
constexpr int GROUP_I = 8;                         // row tiles per band of the tile order
constexpr int64_t kChunk = 32768;                  // backward vocabulary chunk
constexpr uint32_t kOob = 0x80000000u;             // buffer offset that reads as 0
constexpr int kDzLd = BM + 4;   // LDS row (elements) of the staged dZ tile: 520 B, conflict-free
constexpr int kSmemElems = (2 * (BM + BN) * BK > BN * kDzLd) ? 2 * (BM + BN) * BK : BN * kDzLd;

static_assert(BM == BN, "one loader shape serves both operands");

#define LDS_AS __attribute__((address_space(3)))

// An operand of C[i][j] = sum_k P(i, k) Q(j, k), BF16:
//   K-contiguous   (DIM = false): element (d, k) at base[d * ld + k]
//   dim-contiguous (DIM = true):  element (d, k) at base[k * ld + d]
// Reads with d >= dim_limit or k >= k_limit return 0.  Along the contiguous
// axis the test is per 8-element chunk (its first element), so a buffer must
// hold zeros from its limit on that axis up to the next multiple of 8.
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int64_t dim_limit;
  int64_t k_limit;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const uint16_t* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, 0x7fffffff,
                                           0x00020000);
}

// LDS stage of one operand (256 x 64 elements, 32 KB):
//  * K-contiguous: 256 rows (d) of 64 k (128 B, eight 16-byte chunks);
//    logical chunk c of row d sits at c ^ swz(d).
//  * dim-contiguous: two halves (d < 128, d >= 128) of 64 rows (k) of 128 d
//    (256 B, sixteen chunks); logical chunk c of row k sits at c ^ 4 (k & 3).
// Both make the fragment reads below bank-conflict free (measured: a
// transposed read serves 32 lanes, 4 rows x 64 B, per 256-byte bank cycle,
// so the four rows must fall in different 64-byte quarters).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Streams one operand's 256 x 64 slice into an LDS stage.  Load i of wave w
// writes 1 KB at element 2048 w + 512 i of the stage, lane l the 16 bytes at
// 16 l, and each lane reads the logical chunk that lands there:
//  * K-contiguous: rows 32 w + 8 i .. + 7 (lane: row l / 8, chunk l % 8);
//  * dim-contiguous: half w / 4, k rows 16 (w % 4) + 4 i .. + 3 (lane: row
//    l / 16, chunk l % 16).
// So wave w brings rows 32 w .. 32 w + 31 of the tile (K-contiguous) or the
// half w / 4 (dim-contiguous): either way waves 0-3 bring exactly the rows
// 0..127 of P and waves 4-7 the rows 128..255.
template <bool DIM>
struct SliceLoader {
  const uint16_t* tbase;  // operand at the tile's first element, k = 0
  int64_t kstep;          // elements per unit of k
  int64_t k_limit;
  uint32_t off[LD_PER_WAVE];  // byte offset of this lane's 16 bytes, or kOob
  int kc[LD_PER_WAVE];        // k offset (within the slice) this lane's data starts at
  __device__ __forceinline__ void init(const Operand& op, int64_t d0, int wave, int lane) {
    k_limit = op.k_limit;
    if (!DIM) {
      tbase = op.base + d0 * op.ld;
      kstep = 1;
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; ++i) {
        const int row = wave * (BM / 8) + i * ROWS_PER_LD + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        kc[i] = c * 8;
        off[i] = (d0 + row < op.dim_limit) ? (uint32_t)(row * op.ld * 2 + c * 16) : kOob;
      }
    } else {
      tbase = op.base + d0;
      kstep = op.ld;
      const int half = wave >> 2;
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; ++i) {
        const int krow = 16 * (wave & 3) + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (4 * (krow & 3));
        const int d = 128 * half + 8 * c;
        kc[i] = krow;
        off[i] = (d0 + d < op.dim_limit) ? (uint32_t)(krow * op.ld * 2 + d * 2) : kOob;
      }
    }
  }
  // load i of the slice starting at k0; `tail`: the slice reaches past k_limit
  __device__ __forceinline__ void issue(uint16_t LDS_AS* stage, int64_t k0, int wave, int i,
                                        bool tail) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_at(tbase + k0 * kstep);
    uint32_t o = off[i];
    if (tail) o = (k0 + kc[i] < k_limit) ? o : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (void LDS_AS*)(stage + 2048 * wave + 512 * i), 16, o, 0, 0, 0);
  }
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// MFMA operand of the 32 tile rows d0 .. d0 + 31 (d0 a multiple of 32) for
// k-step ks (k = 16 ks .. 16 ks + 15): lane l gets row d0 + l % 32 and the 8 k
// values from 16 ks + 8 (l / 32).
template <bool DIM>
__device__ __forceinline__ bf16x8_t frag(const uint16_t LDS_AS* s, int d0, int ks, int lane) {
  if (!DIM) {
    const int row = d0 + (lane & 31), chunk = 2 * ks + (lane >> 5);
    return __builtin_bit_cast(
        bf16x8_t,
        *reinterpret_cast<const u32x4_t LDS_AS*>(s + row * BK + ((chunk ^ swz(row)) * 8)));
  } else {
    // ds_read_tr16_b64: in each 16-lane group, lane 4 j + q gives the address
    // of 4 elements (q-th quarter) of source row j; lane i receives element i
    // of rows 0..3.  Rows are k here, so lane i gets 4 consecutive k of
    // column d = base + i; two reads give the 8 k values.
    const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
    const int d = d0 + 16 * (g & 1) + 4 * q;
    const int k = 16 * ks + 8 * (g >> 1) + j;
    const uint16_t LDS_AS* p =
        s + (d >> 7) * 8192 + k * 128 + ((((d & 127) >> 3) ^ (4 * j)) * 8) + (d & 7);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_t LDS_AS*)p);
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_t LDS_AS*)(p + 4 * 128));
    const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{a[0], a[1], b[0], b[1]});
  }
}

// Hardware workgroup id -> (row tile, col tile).
__device__ __forceinline__ void tile_of(int b, int n_ti, int n_tj, int* ti, int* tj) {
  const int n = n_ti * n_tj;
  const int q = n >> 3, rem = n & 7;
  const int x = b & 7, slot = b >> 3;
  const int t = x * q + (x < rem ? x : rem) + slot;  // contiguous range per XCD
  const int band = t / (GROUP_I * n_tj);
  const int in_band = t - band * GROUP_I * n_tj;
  const int left = n_ti - band * GROUP_I;
  const int gi = left < GROUP_I ? left : GROUP_I;
  *ti = band * GROUP_I + in_band % gi;
  *tj = in_band / gi;
}

// Accumulator register r of block (a, b) of a lane holds
//   row i = i0 + 128 wr + 32 a + 8 (r / 4) + 4 (lane / 32) + r % 4
//   col j = j0 + 64 wc + 32 b + lane % 32
// for wavefront (wr, wc) = (wave / 4, wave % 4).
template <class Epi, bool PD, bool QD>
__global__ __launch_bounds__(NT) void gemm_kernel(Operand P, Operand Q, int64_t K, int n_ti,
                                                  int n_tj, typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
  uint16_t LDS_AS* const sp = (uint16_t LDS_AS*)smem;  // P stages: sp + s * BM * BK
  uint16_t LDS_AS* const sq = sp + 2 * BM * BK;         // Q stages: sq + s * BN * BK

  int ti, tj;
  tile_of(blockIdx.x, n_ti, n_tj, &ti, &tj);
  const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;

  f32x16_t acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  SliceLoader<PD> lp;
  SliceLoader<QD> lq;
  lp.init(P, i0, wave, lane);
  lq.init(Q, j0, wave, lane);
  const int nk = (int)((K + BK - 1) / BK);
  {
    const bool tail = BK > K;
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) {
      lp.issue(sp, 0, wave, i, tail);
      lq.issue(sq, 0, wave, i, tail);
    }
  }
  // Ping-pong: the two wavefronts of a SIMD (waves w and w + 4) alternate
  // between a memory phase (fragment reads of a half slice, plus the next
  // slice's loads) and a compute phase (16 MFMAs back to back), so one issues
  // LDS and load instructions while the other keeps the matrix core busy.
  // Phases end at workgroup barriers; the second group starts one phase late.
  //   group 0: phase 4k = M(k,0), 4k+1 = C(k,0), 4k+2 = M(k,1), 4k+3 = C(k,1)
  //   group 1: one phase later.
  // Wave w loads rows 32w..32w+31 of both operands, so the P rows a group
  // loads are read by that group only; Q rows are read by both.
  //  * Q rows of slice k+1 go into the stage slice k-1 used, in M(k,0), after
  //    its last readers (group 0 in 4k-2, group 1 in 4k-1).
  //  * P rows of slice k+2 go into the stage of slice k, in M(k,1), right
  //    after the group's own last reads of them (lgkmcnt(0) first): two
  //    phases earlier than M(k+1,0), which gives those loads more time.
  // Group 0 reads slice k+1 from phase 4k+4: at the end of 4k+3 each wave
  // waits until only its four P loads of slice k+2 are in flight
  // (vmcnt(4)), which covers its Q loads of slice k+1 and the P loads of
  // slice k+1 issued before them.
  // Every wave passes the same number of barriers (group 0 adds one at the
  // end), so no barrier waits on a wave that has left the loop.
  const bool g1 = wave >= 4;
  if (nk > 1) {  // P rows of slice 1 (its Q rows follow in M(0,0))
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) lp.issue(sp + BM * BK, BK, wave, i, 2 * BK > K);
  }
  // slice 0 complete (only the P loads of slice 1 may be in flight)
  if (nk > 1)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (g1) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint16_t LDS_AS* cp = sp + cur * BM * BK;
    const uint16_t LDS_AS* cq = sq + cur * BN * BK;
    uint16_t LDS_AS* np = sp + (cur ^ 1) * BM * BK;
    uint16_t LDS_AS* nq = sq + (cur ^ 1) * BN * BK;
    const bool more = kt + 1 < nk;
    const int64_t kn = (int64_t)(kt + 1) * BK;
    const bool tail = kn + BK > K;
    const bool more2 = kt + 2 < nk;
    const int64_t kn2 = (int64_t)(kt + 2) * BK;
    const bool tail2 = kn2 + BK > K;
    uint16_t LDS_AS* cpw = sp + cur * BM * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // memory phase: fragments of k-steps 2h and 2h+1; the next slice's loads
      bf16x8_t fa[2][4], fb[2][NB];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int ks = 2 * h + s2;
#pragma unroll
        for (int a = 0; a < 4; ++a) fa[s2][a] = frag<PD>(cp, wr * 128 + 32 * a, ks, lane);
#pragma unroll
        for (int b = 0; b < NB; ++b) fb[s2][b] = frag<QD>(cq, wc * WN + 32 * b, ks, lane);
      }
      if (h == 0 && more) {
#pragma unroll
        for (int i = 0; i < LD_PER_WAVE; ++i) lq.issue(nq, kn, wave, i, tail);
      }
      // reads complete: the stage may be refilled (now by this wave, after
      // the barrier by the others)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (h == 1) {
        if (more2) {
#pragma unroll
          for (int i = 0; i < LD_PER_WAVE; ++i) lp.issue(cpw, kn2, wave, i, tail2);
        }
        if (g1) {
          if (more2)
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // compute phase
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s2][a], fb[s2][b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // the wait stays behind the MFMAs
      if (h == 1 && !g1) {
        if (more2)
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (!g1) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // LDS is free for the epilogue
  Epi::apply(ep, acc, i0, j0, wr, wc, lane, smem);
}

// ---- epilogues ------------------------------------------------------------------

// Plain FP32 store (the exported building block).
struct EpiF32 {
  struct Params {
    float* C;
    int64_t ldc, rows, cols;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
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
// (max, sum exp(z - max), sum z, sum exp(z - max) (z - max) log2(e)) into the
// partial arrays (the last one gives the entropy), plus the target logit
// written by the one lane that holds it.
struct EpiLse {
  struct Params {
    float* pm;
    float* pd;
    float* ps;
    float* pw;
    float* zt;
    const int64_t* targets;
    int64_t M, V, Mp, ignore_idx;
    int64_t v0;  // vocabulary index of W's first row (0 unless sharded)
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t* smem) {
    float* sh = reinterpret_cast<float*>(smem);  // [wr][wc][b][lane 0..31][4]
    const int64_t vbase = i0 + wr * 128 + 4 * (lane >> 5);
    // rows at offsets >= lim from vbase lie beyond the vocabulary
    const int64_t lim64 = p.V - vbase;
    const int lim = lim64 > 128 ? 128 : (lim64 < 0 ? 0 : (int)lim64);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      float mx = kNegInf;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (a * 32 + 8 * (r >> 2) + (r & 3) < lim) mx = fmaxf(mx, acc[a][b][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mref = (mx == kNegInf) ? 0.0f : mx;
      const float mL = mref * kLog2e;
      float d = 0.0f, s = 0.0f, w = 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (a * 32 + 8 * (r >> 2) + (r & 3) < lim) {
            const float t = __builtin_fmaf(acc[a][b][r], kLog2e, -mL);
            const float e = exp2_hw(t);
            d += e;
            w = __builtin_fmaf(e, t, w);
            s += acc[a][b][r];
          }
      d += __shfl_xor(d, 32, 64);
      s += __shfl_xor(s, 32, 64);
      w += __shfl_xor(w, 32, 64);
      // Target logit: the lane holding row t picks it with a two-level select
      // (row block a, then register r), no dynamic register index.
      if (j < p.M) {
        const int64_t t = p.targets[j];
        const int64_t tl64 = t - p.v0 - vbase;
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
        float* e = sh + (((wr * 4 + wc) * NB + b) * 32 + lane) * 4;
        e[0] = mx;
        e[1] = d;
        e[2] = s;
        e[3] = w;
      }
    }
    __syncthreads();
    // the wavefront of the first vocabulary half merges the second half's state
    if (wr == 0 && lane < 32) {
      const int64_t vt = i0 / BM;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t j = j0 + wc * WN + b * 32 + lane;
        const float* e0 = sh + (((0 * 4 + wc) * NB + b) * 32 + lane) * 4;
        const float* e1 = sh + (((1 * 4 + wc) * NB + b) * 32 + lane) * 4;
        LseEntState st{e0[0], e0[1], e0[2], e0[3]};
        lse_merge(st, LseEntState{e1[0], e1[1], e1[2], e1[3]});
        if (j < p.M) {
          p.pm[vt * p.Mp + j] = st.m;
          p.pd[vt * p.Mp + j] = st.d;
          p.ps[vt * p.Mp + j] = st.s;
          p.pw[vt * p.Mp + j] = st.w;
        }
      }
    }
  }
};

// Backward dZ: rows = vocabulary of the chunk, cols = tokens.
// dZ = g (exp(z - lse) - (1-eps)[v = t] - eps/V), BF16, written token-major
// (dz[m * ldz + v]); padding rows and columns receive zeros.  The dW GEMM
// reads it dim-contiguous, the dX GEMM K-contiguous.  The tile is staged in
// LDS as [token][vocabulary] (rows padded to 520 B: the 8-byte writes of 32
// consecutive tokens hit distinct banks) and leaves as whole 512-byte token
// rows, 16 bytes per lane (direct 8-byte stores from the MFMA layout left
// partial lines: 1.6x the bytes written, measured).
struct EpiDz {
  struct Params {
    uint16_t* dz;
    int64_t ldz, c0, vc_valid;
    const float* stats;
    const int64_t* targets;
    const float* grad_output;
    const int32_t* n_valid;
    const float* entropy;       // with grad_entropy: the forward's entropy
    const float* grad_entropy;  // optional: adds grad_entropy[m] dH/dz
    float eps;
    int reduce_loss;
    int64_t ignore_idx, M, V;
    int64_t v0, Vg;  // W holds vocabulary rows v0 .. v0 + V - 1 of Vg (0, V unless sharded)
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t* smem) {
    uint16_t LDS_AS* const st = (uint16_t LDS_AS*)smem;  // [256 tokens][kDzLd]
    float gscale = 0.0f;
    if (p.reduce_loss) {
      const int32_t nv = p.n_valid[0];
      gscale = p.grad_output[0] / (float)(nv > 0 ? nv : 1);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      int64_t t = -1;
      float g = 0.0f, lse2 = 0.0f;
      bool live = false, bad = false;
      float gH = 0.0f, ez = 0.0f;
      if (j < p.M) {
        t = p.targets[j];
        if (t != p.ignore_idx) {
          if (t >= 0 && t < p.Vg) {
            live = true;
            g = p.reduce_loss ? gscale : p.grad_output[j];
            const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(p.stats + 4 * j);
            lse2 = sv[0] * kLog2e + log2_hw(sv[1]);
            if (p.grad_entropy) {  // dH/dz_v = p_v (E_p[z] - z_v), E_p[z] = lse - H
              gH = p.grad_entropy[j];
              ez = lse2 * kLn2 - p.entropy[j];
            }
          } else {
            bad = true;
          }
        }
      }
      const float goff = g * (p.eps / (float)p.Vg);
      const float gt = g * (1.0f - p.eps);
      // Offsets relative to this lane's first row keep the per-element tests
      // in 32-bit compares against constants.
      const int64_t vrow0 = i0 + wr * 128 + 4 * (lane >> 5);  // chunk-local row of r = 0
      const int64_t tr64 = t - p.v0 - p.c0 - vrow0;
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
            const float z = acc[a][b][4 * q + e];
            float x = exp2_hw(__builtin_fmaf(z, kLog2e, -lse2)) * __builtin_fmaf(gH, ez - z, g) - goff;
            x = (off == trel) ? x - gt : x;
            val[e] = (live && off < lim) ? x : fill;
          }
          const uint32_t w01 = pack_bf16x2(val[0], val[1]), w23 = pack_bf16x2(val[2], val[3]);
          const int jl = wc * WN + b * 32 + (lane & 31);
          const int vl = wr * 128 + 4 * (lane >> 5) + a * 32 + 8 * q;
          *reinterpret_cast<u32x2_t LDS_AS*>(st + jl * kDzLd + vl) = u32x2_t{w01, w23};
        }
    }
    __syncthreads();
    // 256 token rows x 32 chunks of 16 B; 512 threads, consecutive threads
    // take consecutive chunks of a row
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int u = 0; u < (BN * BM / 8) / NT; ++u) {
      const int idx = u * NT + tid, jl = idx >> 5, ch = idx & 31;
      const u32x4_t w = *reinterpret_cast<const u32x4_t LDS_AS*>(st + jl * kDzLd + ch * 8);
      *reinterpret_cast<u32x4_t*>(p.dz + (j0 + jl) * p.ldz + i0 + ch * 8) = w;
    }
  }
};

// Backward dW of a chunk: rows = hidden (h), cols = vocabulary of the chunk.
struct EpiDw {
  struct Params {
    uint16_t* dW;
    int64_t H, c0, vc_valid;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
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
  __device__ static void apply(const Params& p, f32x16_t (&acc)[4][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
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

// ---- merge ------------------------------------------------------------------------

// Per-token merge of the forward partials (fixed order), then loss and stats.
struct MergeParams {
  const float* pm;
  const float* pd;
  const float* ps;
  const float* pw;
  const float* zt;
  const int64_t* targets;
  int64_t M, Mp, V, n_vt, ignore_idx;
  float eps;
  float* loss_tok;
  float* stats;
  float* entropy;  // optional
  int64_t v0;      // vocabulary index of W's first row (0 unless sharded)
  float* partial;  // shard mode: (M, 4) = (m, d, sum z, z_t or 0) instead of loss/stats
};

__global__ __launch_bounds__(256) void lce_merge_kernel(MergeParams p) {
  __shared__ LseEntState sh[8][32];
  const int tl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + tl;
  LseEntState st = {kNegInf, 0.0f, 0.0f, 0.0f};
  if (j < p.M) {
    for (int64_t vt = grp; vt < p.n_vt; vt += 8) {
      const int64_t o = vt * p.Mp + j;
      lse_merge(st, LseEntState{p.pm[o], p.pd[o], p.ps[o], p.pw[o]});
    }
  }
  sh[grp][tl] = st;
  __syncthreads();
  if (grp != 0 || j >= p.M) return;
  for (int g = 1; g < 8; ++g) lse_merge(st, sh[g][tl]);
  const int64_t t = p.targets[j];
  if (p.partial) {  // one vocabulary shard: local statistics for a later merge
    f32x4_t q = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t != p.ignore_idx) {
      const int64_t c = t - p.v0;
      q = f32x4_t{st.m, st.d, st.s, (c >= 0 && c < p.V) ? p.zt[j] : 0.0f};
    }
    *reinterpret_cast<f32x4_t*>(p.partial + 4 * j) = q;
    return;
  }
  if (t == p.ignore_idx) {
    p.loss_tok[j] = 0.0f;
    *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.entropy) p.entropy[j] = 0.0f;
    return;
  }
  if (p.entropy) p.entropy[j] = entropy_of(st.d, st.w);
  const bool t_ok = t >= 0 && t < p.V;
  const float zt = t_ok ? p.zt[j] : __builtin_nanf("");
  const float mean = st.s / (float)p.V;
  const float loss = ce_row_loss(st.m, st.d, zt, mean, p.eps);
  p.loss_tok[j] = t_ok ? loss : __builtin_nanf("");
  *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{st.m, st.d, zt, mean};
}

// ---- host side ------------------------------------------------------------------

template <class Epi, bool PD, bool QD>
hipError_t run_gemm(const Operand& P, const Operand& Q, int64_t rows, int64_t cols, int64_t K,
                    const typename Epi::Params& ep, hipStream_t stream) {
  const int64_t n_ti = (rows + BM - 1) / BM, n_tj = (cols + BN - 1) / BN;
  const int64_t n = n_ti * n_tj;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX / 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<Epi, PD, QD>), dim3((unsigned)n), dim3(NT), 0, stream, P, Q, K,
                     (int)n_ti, (int)n_tj, ep);
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool lce_make_plan(int64_t M, int64_t H, int64_t V, LcePlan* plan) {
  if (M < 0 || H <= 0 || V <= 0 || H % 8 != 0) return false;
  // Every buffer offset a GEMM load forms (256 rows x leading dimension x 2 B)
  // stays below 2^31.
  if (H > ((int64_t)1 << 20) || V > ((int64_t)1 << 31)) return false;
  LcePlan p;
  p.M = M;
  p.H = H;
  p.V = V;
  p.Mp = ((M > 0 ? M : 1) + BN - 1) / BN * BN;
  if (p.Mp > ((int64_t)1 << 22) - BN) return false;
  p.n_vtiles = (V + BM - 1) / BM;
  const int64_t vr = (V + BM - 1) / BM * BM;
  p.chunk = vr < kChunk ? vr : kChunk;
  p.n_chunks = (V + p.chunk - 1) / p.chunk;
  p.ldz = p.chunk;
  const size_t part = align256((size_t)p.n_vtiles * p.Mp * 4);
  const size_t fwd = 4 * part + align256((size_t)p.Mp * 4);
  // backward: dZ of one chunk (Mp x chunk, token-major) and the dX accumulator
  const size_t dz = align256((size_t)p.Mp * p.chunk * 2);
  const size_t dx = p.n_chunks > 1 ? align256((size_t)p.Mp * H * 4) : 0;
  p.off_part = 0;
  p.off_dz = 0;
  p.off_dx = dz;
  const size_t bwd = p.off_dx + dx;
  p.total = fwd > bwd ? fwd : bwd;
  *plan = p;
  return true;
}

hipError_t launch_lce_forward(const LcePlan& plan, const LceFwdArgs& a, hipStream_t stream) {
  const size_t part = align256((size_t)plan.n_vtiles * plan.Mp * 4);
  float* pm = reinterpret_cast<float*>(a.ws + plan.off_part);
  float* pd = reinterpret_cast<float*>(a.ws + plan.off_part + part);
  float* ps = reinterpret_cast<float*>(a.ws + plan.off_part + 2 * part);
  float* pw = reinterpret_cast<float*>(a.ws + plan.off_part + 3 * part);
  float* zt = reinterpret_cast<float*>(a.ws + plan.off_part + 4 * part);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  Operand P{W, plan.H, plan.V, plan.H};
  Operand Q{X, plan.H, plan.M, plan.H};
  EpiLse::Params ep{pm, pd, ps, pw, zt, a.targets, plan.M, plan.V, plan.Mp, a.ignore_idx, a.v0};
  hipError_t e = run_gemm<EpiLse, false, false>(P, Q, plan.V, plan.Mp, plan.H, ep, stream);
  if (e != hipSuccess) return e;
  MergeParams mp{pm, pd, ps, pw, zt, a.targets, plan.M, plan.Mp, plan.V, plan.n_vtiles,
                 a.ignore_idx, a.eps, a.loss_tok, a.stats, a.entropy, a.v0, a.partial};
  hipLaunchKernelGGL(lce_merge_kernel, dim3((unsigned)((plan.M + 31) / 32)), dim3(256), 0, stream,
                     mp);
  return hipGetLastError();
}

// Zero n 16-byte words (dW of an empty batch).
__global__ __launch_bounds__(256) void lce_zero_kernel(u32x4_t* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = u32x4_t{0u, 0u, 0u, 0u};
}

hipError_t launch_lce_backward(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream) {
  if (plan.M == 0) {  // no token: dW = 0 (H is a multiple of 8, dW 16-byte aligned)
    const int64_t n = plan.V * plan.H / 8;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(lce_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<u32x4_t*>(a.dW), n);
    return hipGetLastError();
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(a.ws + plan.off_dz);
  float* dxacc = reinterpret_cast<float*>(a.ws + plan.off_dx);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  for (int64_t c = 0; c < plan.n_chunks; ++c) {
    const int64_t c0 = c * plan.chunk;
    const int64_t vc = (plan.V - c0) < plan.chunk ? (plan.V - c0) : plan.chunk;
    const uint16_t* Wc = W + c0 * plan.H;
    // dZ of the chunk: (vocabulary x tokens), K = H, both operands K-contiguous
    {
      Operand P{Wc, plan.H, vc, plan.H};
      Operand Q{X, plan.H, plan.M, plan.H};
      EpiDz::Params ep{dz, plan.ldz, c0, vc, a.stats, a.targets, a.grad_output, a.n_valid,
                       a.entropy, a.grad_entropy, a.eps, a.reduce_loss, a.ignore_idx, plan.M,
                       plan.V, a.v0, a.Vg};
      hipError_t e = run_gemm<EpiDz, false, false>(P, Q, vc, plan.Mp, plan.H, ep, stream);
      if (e != hipSuccess) return e;
    }
    // dW rows of the chunk: (hidden x vocabulary), K = tokens; X (h contiguous
    // per token) and dZ (v contiguous per token) are both read dim-contiguous
    {
      Operand P{X, plan.H, plan.H, plan.M};
      Operand Q{dz, plan.ldz, vc, plan.M};
      EpiDw::Params ep{static_cast<uint16_t*>(a.dW), plan.H, c0, vc};
      hipError_t e = run_gemm<EpiDw, true, true>(P, Q, plan.H, vc, plan.M, ep, stream);
      if (e != hipSuccess) return e;
    }
    // dX += dZ_c W_c: (hidden x tokens), K = vocabulary of the chunk; W_c is
    // read dim-contiguous (h contiguous per vocabulary row), dZ K-contiguous
    {
      Operand P{Wc, plan.H, plan.H, vc};
      Operand Q{dz, plan.ldz, plan.M, vc};
      const int mode = (c > 0 ? 1 : 0) | (c + 1 == plan.n_chunks ? 2 : 0);
      EpiDx::Params ep{dxacc, static_cast<uint16_t*>(a.dX), plan.H, plan.M, mode};
      hipError_t e = run_gemm<EpiDx, true, false>(P, Q, plan.H, plan.M, vc, ep, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const void* P, int64_t ldp, int p_dim, const void* Q, int64_t ldq,
                            int q_dim, int64_t rows, int64_t cols, int64_t K, float* C,
                            int64_t ldc, hipStream_t stream) {
  Operand op{static_cast<const uint16_t*>(P), ldp, rows, K};
  Operand oq{static_cast<const uint16_t*>(Q), ldq, cols, K};
  EpiF32::Params ep{C, ldc, rows, cols};
  if (!p_dim && !q_dim) return run_gemm<EpiF32, false, false>(op, oq, rows, cols, K, ep, stream);
  if (!p_dim && q_dim) return run_gemm<EpiF32, false, true>(op, oq, rows, cols, K, ep, stream);
  if (p_dim && !q_dim) return run_gemm<EpiF32, true, false>(op, oq, rows, cols, K, ep, stream);
  return run_gemm<EpiF32, true, true>(op, oq, rows, cols, K, ep, stream);
}

}  // namespace vce
