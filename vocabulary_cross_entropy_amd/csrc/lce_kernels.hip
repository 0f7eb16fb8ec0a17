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
//  * One GEMM core, C[i][j] = sum_k P(i, k) Q(j, k), each operand stored
//    K-contiguous or dim-contiguous (a template flag), so the backward reads
//    X, W and dZ where they lie.  A 256 x 256 output tile per 256-thread
//    workgroup: four wavefronts, one per SIMD, of 128 x 128 each
//    (v_mfma_f32_32x32x16_bf16, 16 accumulator blocks = all 256 AGPRs).  A
//    wave tile this size reads a third fewer LDS bytes per flop than two
//    waves of 128 x 64 per SIMD.
//  * K advances in 64-deep slices through two LDS stages (128 KB of 160 KB).
//    Operands travel global -> VGPRs -> LDS: every wave keeps two slices in
//    flight in two register buffers (64 VGPRs each), so each 16-byte load is
//    issued two slices before its data is written to LDS.  The 16 loads and
//    16 LDS writes of a wave per slice are spread evenly, one pair every
//    three MFMAs (loads issued in one burst after each barrier, as with
//    direct-to-LDS loads into two stages, left the MFMAs waiting: measured
//    1150-1200 TFLOP/s against 1470-1600 with the loads taken out).
//  * One barrier per slice, two MFMAs into its last k-step (those two keep
//    the MFMA pipe busy while the wave waits): it publishes the next slice's
//    LDS writes and frees the stage just read.  The fragment reads of the
//    next k-step go out right after the second MFMA of each k-step, in the
//    order the MFMAs consume them.
//  * Tile order: hardware workgroup ids go round-robin over the 8 XCDs, so
//    each XCD is given a contiguous range of tiles, walked in bands of 8 row
//    tiles so the 32 workgroups an XCD runs at once share both operands in
//    its L2.
//  * Forward: tiles are (vocabulary x tokens); each lane owns tokens, so the
//    epilogue reduces the online LSE (max, sum of exp, sum of logits) over the
//    vocabulary inside the lane, then across the two lane halves and the two
//    wavefronts that share the tokens.  Per-tile partials are merged per
//    token by a second kernel in a fixed order.
//  * Backward, per vocabulary chunk: recompute the logits and write dZ (BF16,
//    token-major) straight from the accumulators (a lane swap turns the MFMA
//    layout into 16-byte pieces of token rows; staging the tile in LDS and
//    storing whole rows was measured slower); dW rows of the chunk are
//    finished by one GEMM over all tokens (written once, never accumulated);
//    dX accumulates chunk by chunk in FP32, the last chunk writes BF16.
#include <type_traits>

#include "vce_device.h"
#include "vce_internal.h"

namespace vce {

namespace {

constexpr int BM = 256;   // output rows per tile (P side)
constexpr int BN = 256;   // output cols per tile (Q side)
constexpr int BK = 64;    // K slice per stage
constexpr int NT = 256;   // threads per workgroup: 4 wavefronts, one per SIMD
constexpr int WM = 128;   // output rows per wavefront
constexpr int WN = 128;   // output cols per wavefront
constexpr int NA = WM / 32;                        // 32-row blocks per wavefront (4)
constexpr int NB = WN / 32;                        // 32-column blocks per wavefront (4)
constexpr int NWC = BN / WN;                       // wavefronts across the columns (2)
constexpr int UNITS = BM * BK * 2 / 1024;          // 1 KB units per operand per slice (32)
constexpr int UPW = UNITS / (NT / 64);             // units per wave per operand (8)
constexpr int GROUP_I = 8;                         // row tiles per band of the tile order
constexpr int64_t kChunk = 32768;                  // backward vocabulary chunk
constexpr uint32_t kOob = 0x80000000u;             // buffer offset that reads as 0
constexpr int kSmemElems = 2 * (BM + BN) * BK;  // two stages of both operands (128 KB)

static_assert(BM == BN, "one loader shape serves both operands");
static_assert(NA == 4 && NB == 4 && UPW == 8, "the schedule below assumes these");

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

// LDS stage of one operand (256 x 64 elements, 32 KB, 32 units of 1 KB):
//  * K-contiguous: 256 rows (d) of 64 k (128 B, eight 16-byte chunks);
//    logical chunk c of row d sits at c ^ swz(d).
//  * dim-contiguous: two halves (d < 128, d >= 128) of 64 rows (k) of 128 d
//    (256 B, sixteen chunks); logical chunk c of row k sits at c ^ 4 (k & 3).
// Both make the fragment reads below bank-conflict free (measured: a
// transposed read serves 32 lanes, 4 rows x 64 B, per 256-byte bank cycle,
// so the four rows must fall in different 64-byte quarters).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Moves one operand's 256 x 64 slices in 1 KB units, 8 per wave: unit q =
// 8 w + i of wave w, lane l, 16 bytes each.  All that varies with i is a
// scalar offset of the global read and an immediate (or one XOR) of the LDS
// write, so a loader holds two VGPRs:
//  * K-contiguous: rows 8 q .. 8 q + 7, lane l reads logical chunk l % 8 of
//    row 8 q + l / 8 and writes it at physical chunk (l % 8) ^ swz(row) =
//    (l % 8) ^ (l / 8) ^ i.  Rows past dim_limit are cut off by the buffer
//    size; with MASK, chunks at or past k_limit by an out-of-range offset.
//  * dim-contiguous: half q / 16 (= w / 2), k rows 4 (q % 16) + l / 16, lane
//    chunk l % 16 read from logical chunk (l % 16) ^ 4 (l / 16 % 4) of that
//    row and written at 16 l of the unit.  Columns past dim_limit get an
//    out-of-range offset; k rows past k_limit are cut off by the buffer size.
// at(k0) gives the slice's buffer (scalar, once per slice); get() loads a
// unit into registers, put() writes registers to the stage; direct() loads a
// unit of the first slice straight into LDS (the prologue).
struct SliceRef {
  __amdgpu_buffer_rsrc_t rs;
  int nv;  // K-contiguous with MASK: chunks (of 8 k) of the slice below k_limit, 0..8
};

template <bool DIM>
struct SliceLoader {
  const uint16_t* tbase;  // operand at the tile's first element, k = 0
  int64_t ld;
  int64_t k_limit;
  int64_t rows_bytes;  // K-contiguous: bytes of the tile's rows below dim_limit
  uint32_t voff;       // this lane's byte offset in unit 0, or kOob
  uint32_t ustep;      // bytes between the sources of consecutive units
  int lds;             // element offset of this lane's 16 bytes of unit 0 in a stage
  int kch;             // K-contiguous: the logical chunk this lane reads (l % 8)
  __device__ __forceinline__ void init(const Operand& op, int64_t d0, int wave, int lane) {
    k_limit = op.k_limit;
    ld = op.ld;
    if (!DIM) {
      tbase = op.base + d0 * op.ld;
      const int64_t rl = op.dim_limit - d0;
      rows_bytes = rl <= 0 ? 0 : rl * op.ld * 2;
      const int row = 8 * UPW * wave + (lane >> 3);
      voff = (uint32_t)(row * op.ld * 2 + (lane & 7) * 16);
      ustep = (uint32_t)__builtin_amdgcn_readfirstlane((int)(8 * op.ld * 2));
      kch = lane & 7;
      const int c0 = ((lane & 7) ^ (lane >> 3)) & 7;  // physical chunk in unit 0
      lds = row * BK + c0 * 8;                        // unit i: (lds ^ 8 i) + 512 i
    } else {
      tbase = op.base + d0;
      rows_bytes = 0;
      const int krow = 32 * (wave & 1) + (lane >> 4);
      const int c = (lane & 15) ^ (4 * ((lane >> 4) & 3));
      const int d = 128 * (wave >> 1) + 8 * c;
      voff = (d0 + d < op.dim_limit) ? (uint32_t)(krow * op.ld * 2 + d * 2) : kOob;
      ustep = (uint32_t)__builtin_amdgcn_readfirstlane((int)(4 * op.ld * 2));
      kch = 0;
      lds = 512 * UPW * wave + 8 * lane;  // unit i: + 512 i
    }
  }
  // the slice starting at k0 (a multiple of BK, possibly past K).  MASK:
  // reads at or past k_limit give 0.  Without it K is a multiple of 2 BK and
  // the caller clamps slices past the end (prefetched, never used) to the
  // last one.
  template <bool MASK>
  __device__ __forceinline__ SliceRef at(int64_t k0) const {
    SliceRef r;
    r.nv = 8;
    const int64_t kb = k0;
    if (!DIM) {
      r.rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(tbase + kb), (short)0,
          rows_bytes > 0x7fffffff ? 0x7fffffff : (int)rows_bytes, 0x00020000);
      if (MASK) {
        const int64_t left = k_limit - k0;
        r.nv = left <= 0 ? 0 : (left >= BK ? 8 : (int)((left + 7) >> 3));
      }
    } else {
      int64_t bytes = 0x7fffffff;
      if (MASK) {
        const int64_t left = k_limit - k0;
        bytes = left <= 0 ? 0 : left * ld * 2;
        if (bytes > 0x7fffffff) bytes = 0x7fffffff;
      }
      r.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tbase + kb * ld), (short)0,
                                               (int)bytes, 0x00020000);
    }
    return r;
  }
  template <bool MASK>
  __device__ __forceinline__ u32x4_t get(const SliceRef& r, int i) const {
    // K-contiguous: this lane reads logical chunk l % 8, which lies below
    // k_limit iff (l % 8) < nv
    const uint32_t o = (!MASK || DIM || kch < r.nv) ? voff : kOob;
    return __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r.rs, o, (int)(i * ustep), 0));
  }
  __device__ __forceinline__ void put(uint16_t LDS_AS* stage, int i, const u32x4_t& v) const {
    const int e = DIM ? lds + 512 * i : (lds ^ (8 * i)) + 512 * i;
    *reinterpret_cast<u32x4_t LDS_AS*>(stage + e) = v;
  }
  // Unit i straight into LDS: lane l fills the 16 bytes at 16 l of the unit,
  // so a K-contiguous lane reads the logical chunk that sits there,
  // (l % 8) ^ (l / 8) ^ i, instead of l % 8.
  template <bool MASK>
  __device__ __forceinline__ void direct(uint16_t LDS_AS* stage, const SliceRef& r, int wave,
                                         int lane, int i) const {
    uint32_t o = voff;
    if (!DIM) {
      const int c = ((lane & 7) ^ (lane >> 3) ^ i) & 7;
      o = voff - (uint32_t)((lane & 7) * 16) + (uint32_t)(c * 16);
      if (MASK && c >= r.nv) o = kOob;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r.rs, (void LDS_AS*)(stage + 512 * (UPW * wave + i)), 16, o, (int)(i * ustep), 0, 0);
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

// Per-wave state of the main loop.
struct LoopState {
  f32x16_t acc[NA][NB];
  bf16x8_t FA[NA];          // P fragments (refilled for the next k-step as they die)
  bf16x8_t FB[2][NB];       // Q fragments of the current and the next k-step
  u32x4_t R[2][2 * UPW];    // register buffers: units 0..7 of P, 8..15 of Q
};

// Slice k of the main loop (its data in stage k & 1, its first k-step's
// fragments in FA and FB[0]).  During k-steps 0..2 the wave writes slice
// k + 1 from register buffer B1 = (k + 1) & 1 to the other stage and refills
// the buffer with slice k + 3.  The barrier early in k-step 3 (after its
// first two MFMAs, before any read of the other stage) publishes slice k + 1
// (every wave waited for its own writes) and tells that stage k is no longer
// read (every wave's fragments of k-step 3 are in registers), so the next
// round of writes may go there.  MFMAs run a-major: P fragment a dies
// after MFMA 4 a + 3 and is refilled with the next k-step's right then; the
// next Q fragments go to the other buffer after MFMA 1 (MFMA 2 in k-step
// 3, behind the barrier).  Waits: the compiler
// places s_waitcnt vmcnt before each LDS write (its load was issued 32 loads
// earlier) and lgkmcnt before the MFMAs that use fresh fragments.
template <int B1, bool PD, bool QD, bool MASK, bool ZERO = false>
__device__ __forceinline__ void loop_slice(LoopState& S, const SliceLoader<PD>& lp,
                                           const SliceLoader<QD>& lq, uint16_t LDS_AS* sp,
                                           uint16_t LDS_AS* sq, int k, int klast, int wr,
                                           int wc, int lane) {
  constexpr int cur = B1 ^ 1;  // k & 1: the loop runs slices in pairs
  const uint16_t LDS_AS* cp = sp + cur * BM * BK;
  const uint16_t LDS_AS* cq = sq + cur * BN * BK;
  uint16_t LDS_AS* np = sp + (cur ^ 1) * BM * BK;
  uint16_t LDS_AS* nq = sq + (cur ^ 1) * BN * BK;
  const int k3 = MASK || k + 3 < klast ? k + 3 : klast;
  const SliceRef rp = lp.template at<MASK>((int64_t)k3 * BK);
  const SliceRef rq = lq.template at<MASK>((int64_t)k3 * BK);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int f = ks & 1;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int m = a * NB + b;
        // the barrier goes in after two MFMAs of k-step 3 (their operands are
        // in registers), so the MFMA pipe stays busy while the wave waits for
        // its last fragment read and for the other waves
        if (ks == 3 && m == 2) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        // ZERO (the tile's first slice): k-step 0 starts from C = 0, an
        // inline constant of the MFMA, so the accumulators need no clearing
        const f32x16_t c = (ZERO && ks == 0) ? f32x16_t{} : S.acc[a][b];
        S.acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.FA[a], S.FB[f][b], c, 0, 0, 0);
        // next k-step's Q fragments (at k-step 3: of the next slice, from the
        // stage the barrier has just published)
        if (m == (ks == 3 ? 2 : 1)) {
#pragma unroll
          for (int r = 0; r < NB; ++r)
            S.FB[f ^ 1][r] = ks < 3 ? frag<QD>(cq, wc * WN + 32 * r, ks + 1, lane)
                                    : frag<QD>(nq, wc * WN + 32 * r, 0, lane);
        }
        if (b == NB - 1)
          S.FA[a] = ks < 3 ? frag<PD>(cp, wr * WM + 32 * a, ks + 1, lane)
                           : frag<PD>(np, wr * WM + 32 * a, 0, lane);
        const int pos = ks * 16 + m;
        if (ks < 3 && pos % 3 == 2) {
          const int u = pos / 3;  // 0..15
          if (u < UPW) {
            lp.put(np, u, S.R[B1][u]);
            S.R[B1][u] = lp.template get<MASK>(rp, u);
          } else {
            lq.put(nq, u - UPW, S.R[B1][u]);
            S.R[B1][u] = lq.template get<MASK>(rq, u - UPW);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Accumulator register r of block (a, b) of a lane holds
//   row i = i0 + 128 wr + 32 a + 8 (r / 4) + 4 (lane / 32) + r % 4
//   col j = j0 + 128 wc + 32 b + lane % 32
// for wavefront (wr, wc) = (wave / 2, wave % 2).
// One output tile: tile number b of the problem (P, Q, K), then the epilogue.
// MASK: K is not a multiple of 2 BK (or is 0): k is masked on every read.
// Up to three operand pairs whose products one tile sums before its
// epilogue: C[i][j] = sum_s sum_k P_s(i, k) Q_s(j, k), every pair with the
// same K.  One pair is the plain GEMM; three carry the FP32-input form, whose
// operands are each split into two BF16 planes (see split_bf16_kernel).
template <int NSEG>
struct Segs {
  Operand P[NSEG], Q[NSEG];
  // pair s by value (constant indices only, so the kernel arguments are read
  // in place and never copied to scratch)
  __device__ __forceinline__ Operand p(int s) const {
    Operand r = P[0];
#pragma unroll
    for (int t = 1; t < NSEG; ++t)
      if (s == t) r = P[t];
    return r;
  }
  __device__ __forceinline__ Operand q(int s) const {
    Operand r = Q[0];
#pragma unroll
    for (int t = 1; t < NSEG; ++t)
      if (s == t) r = Q[t];
    return r;
  }
};

// One operand pair's sum over K added to the accumulators in S (ZERO: stored
// into them, whatever they held): loaders, prologue and main loop, then a
// drain and a barrier, after which both LDS stages are free again (for the
// next pair or the epilogue).
template <bool PD, bool QD, bool MASK, bool ZERO>
__device__ __forceinline__ void mainloop(LoopState& S, const Operand& P, const Operand& Q,
                                         int64_t K, int64_t i0, int64_t j0, int wave, int lane,
                                         int wr, int wc, uint16_t LDS_AS* sp,
                                         uint16_t LDS_AS* sq) {
  SliceLoader<PD> lp;
  SliceLoader<QD> lq;
  lp.init(P, i0, wave, lane);
  lq.init(Q, j0, wave, lane);
  // Q's stages start 64 KB into LDS, past the 16-bit offset of an LDS
  // instruction; with that base opaque to the compiler, each fragment address
  // of Q is one register for both stages (stage and block go in the offset).
  // Measured on the one-pair tile only (it gave the three-pair tile more
  // spills).
  if (ZERO) asm volatile("" : "+v"(sq));
  // An even number of slices (the loop body runs two); slices at or past K
  // read as zeros and add nothing.
  const int nk = (int)((K + 2 * BK - 1) / (2 * BK)) * 2;
  // last real slice (without MASK, prefetches past it re-read it)
  const int klast = (int)((K + BK - 1) / BK) - 1;
  // slice 0 straight to stage 0, slices 1 and 2 into register buffers 1 and
  // 0 right behind it; then wait for slice 0 only (its 16 loads went first)
  {
    const SliceRef p0 = lp.template at<MASK>(0), q0 = lq.template at<MASK>(0);
#pragma unroll
    for (int i = 0; i < UPW; ++i) lp.template direct<MASK>(sp, p0, wave, lane, i);
#pragma unroll
    for (int i = 0; i < UPW; ++i) lq.template direct<MASK>(sq, q0, wave, lane, i);
    const int k1 = MASK || klast >= 1 ? 1 : klast, k2 = MASK || klast >= 2 ? 2 : klast;
    const SliceRef p1 = lp.template at<MASK>((int64_t)k1 * BK);
    const SliceRef q1 = lq.template at<MASK>((int64_t)k1 * BK);
#pragma unroll
    for (int i = 0; i < UPW; ++i) S.R[1][i] = lp.template get<MASK>(p1, i);
#pragma unroll
    for (int i = 0; i < UPW; ++i) S.R[1][UPW + i] = lq.template get<MASK>(q1, i);
    const SliceRef p2 = lp.template at<MASK>((int64_t)k2 * BK);
    const SliceRef q2 = lq.template at<MASK>((int64_t)k2 * BK);
#pragma unroll
    for (int i = 0; i < UPW; ++i) S.R[0][i] = lp.template get<MASK>(p2, i);
#pragma unroll
    for (int i = 0; i < UPW; ++i) S.R[0][UPW + i] = lq.template get<MASK>(q2, i);
  }
  asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < NA; ++a) S.FA[a] = frag<PD>(sp, wr * WM + 32 * a, 0, lane);
#pragma unroll
  for (int b = 0; b < NB; ++b) S.FB[0][b] = frag<QD>(sq, wc * WN + 32 * b, 0, lane);
  int k = 0;
  if (ZERO) {
    if (nk == 0) {  // K = 0: the sum is empty
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) S.acc[a][b] = f32x16_t{};
    } else {
      loop_slice<1, PD, QD, MASK, true>(S, lp, lq, sp, sq, 0, klast, wr, wc, lane);
      loop_slice<0, PD, QD, MASK>(S, lp, lq, sp, sq, 1, klast, wr, wc, lane);
      k = 2;
    }
  }
  for (; k < nk; k += 2) {
    loop_slice<1, PD, QD, MASK>(S, lp, lq, sp, sq, k, klast, wr, wc, lane);
    loop_slice<0, PD, QD, MASK>(S, lp, lq, sp, sq, k + 1, klast, wr, wc, lane);
  }
  // drain the loads of the slices past the end (zeros, never used) and let
  // every wave finish with LDS before the epilogue (or the next pair) reuses it
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
}

template <class Epi, bool PD, bool QD, bool MASK, int NSEG>
__device__ __forceinline__ void gemm_tile(const Segs<NSEG>& G, int64_t K, int bid, int n_ti,
                                          int n_tj, const typename Epi::Params& ep,
                                          uint16_t* smem) {
  uint16_t LDS_AS* const sp = (uint16_t LDS_AS*)smem;  // P stages: sp + s * BM * BK
  uint16_t LDS_AS* const sq = sp + 2 * BM * BK;         // Q stages: sq + s * BN * BK

  int ti, tj;
  tile_of(bid, n_ti, n_tj, &ti, &tj);
  const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int wr = wave / NWC, wc = wave % NWC;

  LoopState S;
  if (NSEG == 1) {
    // the first k-step writes the accumulators
    mainloop<PD, QD, MASK, true>(S, G.p(0), G.q(0), K, i0, j0, wave, lane, wr, wc, sp, sq);
  } else {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.acc[a][b][r] = 0.0f;
    // one copy of the main loop, run once per pair
#pragma nounroll
    for (int s = 0; s < NSEG; ++s)
      mainloop<PD, QD, MASK, false>(S, G.p(s), G.q(s), K, i0, j0, wave, lane, wr, wc, sp, sq);
  }
  // the epilogue's lane index is computed anew after the loop (from a value
  // the compiler cannot hoist), so no per-lane index lives across the loop
  unsigned z = 0;
  asm volatile("" : "+s"(z));
  const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z));
  Epi::apply(ep, S.acc, i0, j0, wr, wc, elane, smem);
}

template <class Epi, bool PD, bool QD, bool MASK, int NSEG>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(Segs<NSEG> G, int64_t K, int n_ti,
                                                     int n_tj, typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
  gemm_tile<Epi, PD, QD, MASK, NSEG>(G, K, blockIdx.x, n_ti, n_tj, ep, smem);
}

// Two independent problems in one grid, the first one's tiles first: the
// backward's dX and dW GEMMs of a chunk (both read only that chunk's dZ), so
// that the short grid of one fills the last wave of the other.
template <int NSEG>
struct GemmProblem {
  Segs<NSEG> G;
  int64_t K;
  int n_ti, n_tj;
};

template <class EA, bool PA, bool QA, bool MA, class EB, bool PB, bool QB, bool MB, int NSEG>
__global__ __launch_bounds__(NT, 1) void gemm2_kernel(GemmProblem<NSEG> A,
                                                      typename EA::Params ea,
                                                      GemmProblem<NSEG> B,
                                                      typename EB::Params eb) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
  const int na = A.n_ti * A.n_tj;
  if ((int)blockIdx.x < na)
    gemm_tile<EA, PA, QA, MA, NSEG>(A.G, A.K, blockIdx.x, A.n_ti, A.n_tj, ea, smem);
  else
    gemm_tile<EB, PB, QB, MB, NSEG>(B.G, B.K, blockIdx.x - na, B.n_ti, B.n_tj, eb, smem);
}

// Three independent problems in one grid, in this order: the backward's dX and
// dW GEMMs of chunk c (both read that chunk's dZ) and the dZ GEMM of chunk
// c + 1 (written to the other dZ buffer).  The next chunk's short dZ tiles
// fill the last wave of the long dX and dW tiles, which separate launches
// leave partly idle.
template <class EA, bool PA, bool QA, bool MA, class EB, bool PB, bool QB, bool MB, class EC,
          bool PC, bool QC, bool MC, int NSEG>
__global__ __launch_bounds__(NT, 1) void gemm3_kernel(GemmProblem<NSEG> A,
                                                      typename EA::Params ea,
                                                      GemmProblem<NSEG> B,
                                                      typename EB::Params eb,
                                                      GemmProblem<NSEG> C,
                                                      typename EC::Params ec) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
  const int na = A.n_ti * A.n_tj, nb = B.n_ti * B.n_tj;
  const int bid = blockIdx.x;
  if (bid < na)
    gemm_tile<EA, PA, QA, MA, NSEG>(A.G, A.K, bid, A.n_ti, A.n_tj, ea, smem);
  else if (bid < na + nb)
    gemm_tile<EB, PB, QB, MB, NSEG>(B.G, B.K, bid - na, B.n_ti, B.n_tj, eb, smem);
  else
    gemm_tile<EC, PC, QC, MC, NSEG>(C.G, C.K, bid - na - nb, C.n_ti, C.n_tj, ec, smem);
}

// ---- epilogues ------------------------------------------------------------------

// Plain FP32 store (the exported building block).
struct EpiF32 {
  struct Params {
    float* C;
    int64_t ldc, rows, cols;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
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
// Tree reductions of one accumulator block (16 values): short dependency
// chains, since one wavefront per SIMD has no other wave to fill the gaps.
__device__ __forceinline__ float max16(const f32x16_t& v) {
  // three-input maxima (v_max3_f32): 5 + 2 + 1 instructions
  float m[6];
#pragma unroll
  for (int i = 0; i < 5; ++i) m[i] = fmaxf(fmaxf(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
  m[5] = v[15];
  return fmaxf(fmaxf(fmaxf(m[0], m[1]), m[2]), fmaxf(fmaxf(m[3], m[4]), m[5]));
}

// Register (a, r) = (tl / 32, 4 ((tl / 8) % 4) + tl % 4) of a lane's column
// b, for a row offset tl of that lane (bit 2 clear), without a dynamic
// register index: a running select that reads one accumulator at a time
// (used only by the rare lanes that hold a target, so it is kept out of the
// register budget of the common path).
__device__ __forceinline__ float pick(const f32x16_t (&acc)[NA][NB], int b, int tl) {
  const int want = (tl >> 5) * 16 + ((tl >> 3) & 3) * 4 + (tl & 3);
  float z = 0.0f;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) z = (want == a * 16 + r) ? acc[a][b][r] : z;
    __builtin_amdgcn_sched_barrier(0);
  }
  return z;
}

template <bool ENT>
struct EpiLseT {
  struct Params {
    float* pm;
    float* pd;
    float* ps;
    float* pw;
    float* zt;
    const int64_t* targets;
    int64_t M, V, Mp, ignore_idx;
    int64_t v0;  // vocabulary index of W's first row (0 unless sharded)
    float scale;   // logits are scale times the accumulators (1 unscaled)
    float slog2e;  // fl(scale log2(e)), the exponent's factor
  };
  // Sum over the block's values of exp(z - m) (as d), the accumulators (as
  // s) and, with ENT, exp(z - m) (z - m) log2(e) (as w), each as a tree; rows
  // at offsets >= lim left out when MASKED.  z = scale v, so the exponent is
  // v fl(scale log2(e)) - mL.
  template <bool MASKED>
  __device__ static void sums(const f32x16_t& v, int a, float sl2e, float mL, int lim, float& d,
                              float& s, float& w) {
    float e[16], t[16], z[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool in = !MASKED || a * 32 + 8 * (r >> 2) + (r & 3) < lim;
      t[r] = __builtin_fmaf(v[r], sl2e, -mL);
      e[r] = in ? exp2_hw(t[r]) : 0.0f;
      z[r] = in ? v[r] : 0.0f;
      if (ENT) t[r] = in ? e[r] * t[r] : 0.0f;
    }
#pragma unroll
    for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
      for (int r = 0; r < h; ++r) {
        e[r] += e[r + h];
        z[r] += z[r + h];
        if (ENT) t[r] += t[r + h];
      }
    d += e[0];
    s += z[0];
    if (ENT) w += t[0];
  }
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t* smem) {
    float* sh = reinterpret_cast<float*>(smem);  // [wr][wc][b][lane 0..31][4]
    // the lane's four targets first: one memory round trip under the math
    int64_t tg[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      tg[b] = j < p.M ? p.targets[j] : p.ignore_idx;
    }
    const int64_t vbase = i0 + wr * 128 + 4 * (lane >> 5);
    // rows at offsets >= lim from vbase lie beyond the vocabulary; a wave
    // whose 128 rows are all inside skips every per-element test
    const bool full = p.V - (i0 + wr * 128) >= 128;
    const int64_t lim64 = p.V - vbase;
    const int lim = lim64 > 128 ? 128 : (lim64 < 0 ? 0 : (int)lim64);
    // one token column at a time (the scheduling barriers keep the columns
    // apart, so the accumulator copies of one column are live at once)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float mx;
      if (full) {
        mx = fmaxf(fmaxf(max16(acc[0][b]), max16(acc[1][b])),
                   fmaxf(max16(acc[2][b]), max16(acc[3][b])));
      } else {
        mx = kNegInf;
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (a * 32 + 8 * (r >> 2) + (r & 3) < lim) mx = fmaxf(mx, acc[a][b][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mL = ((mx == kNegInf) ? 0.0f : mx) * p.slog2e;
      float d = 0.0f, sz = 0.0f, w = 0.0f;
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        if (full)
          sums<false>(acc[a][b], a, p.slog2e, mL, lim, d, sz, w);
        else
          sums<true>(acc[a][b], a, p.slog2e, mL, lim, d, sz, w);
        __builtin_amdgcn_sched_barrier(0);  // one block's temporaries at a time
      }
      d += __shfl_xor(d, 32, 64);
      sz += __shfl_xor(sz, 32, 64);
      if (ENT) w += __shfl_xor(w, 32, 64);
      // Every term above carries the factor 2^rho of the rounding rho =
      // m log2(e) - mL (exact by an FMA), and every exponent t the addend rho:
      // taken back out of the column's sums, d -> 2^-rho d and
      // w -> 2^-rho (w - rho d), so the error of a term does not grow with |m|
      // (up to |m| of about 2^29, where 2^rho would leave the FP32 range).
      {
        const float rho = __builtin_fmaf((mx == kNegInf) ? 0.0f : mx, p.slog2e, -mL);
        // 2^-rho - 1 = -rho ln 2 to within (rho ln 2)^2 / 2 for |rho| < 2^-10
        // (|m| < 2^13); beyond, the exponential, on a branch the whole
        // wavefront skips in the common case
        float corr = -rho * kLn2;
        if (__builtin_amdgcn_ballot_w64(!(fabsf(rho) < 0x1p-10f)))
          corr = fabsf(rho) < 0x1p-10f ? corr : exp2_hw(-rho) - 1.0f;
        if (ENT) w = __builtin_fmaf(__builtin_fmaf(-rho, d, w), corr, __builtin_fmaf(-rho, d, w));
        d = __builtin_fmaf(d, corr, d);
      }
      // Target logit: only a lane whose token's target lies in this wave's
      // rows (rarely any) picks it.
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      {
        const int64_t t = tg[b];
        const int64_t tl64 = t - p.v0 - vbase;
        const bool inr = t != p.ignore_idx && tl64 >= 0 && tl64 < 128 && ((tl64 >> 2) & 1) == 0;
        if (inr) p.zt[j] = p.scale * pick(acc, b, (int)tl64);
      }
      if (lane < 32) {
        float* e = sh + (((wr * NWC + wc) * NB + b) * 32 + lane) * 4;
        // the maximum and the sum of logits in logit units (scale times the
        // accumulators; d and w are relative to that maximum already)
        *reinterpret_cast<f32x4_t*>(e) = f32x4_t{p.scale * mx, d, p.scale * sz, w};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // the wavefront of the first vocabulary half merges the second half's state
    if (wr == 0 && lane < 32) {
      const int64_t vt = i0 / BM;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t j = j0 + wc * WN + b * 32 + lane;
        const f32x4_t e0 =
            *reinterpret_cast<const f32x4_t*>(sh + (((0 * NWC + wc) * NB + b) * 32 + lane) * 4);
        const f32x4_t e1 =
            *reinterpret_cast<const f32x4_t*>(sh + (((1 * NWC + wc) * NB + b) * 32 + lane) * 4);
        if (j >= p.M) continue;
        if (ENT) {
          LseEntState st{e0[0], e0[1], e0[2], e0[3]};
          lse_merge(st, LseEntState{e1[0], e1[1], e1[2], e1[3]});
          p.pm[vt * p.Mp + j] = st.m;
          p.pd[vt * p.Mp + j] = st.d;
          p.ps[vt * p.Mp + j] = st.s;
          p.pw[vt * p.Mp + j] = st.w;
        } else {
          LseState st{e0[0], e0[1], e0[2]};
          lse_merge(st, LseState{e1[0], e1[1], e1[2]});
          p.pm[vt * p.Mp + j] = st.m;
          p.pd[vt * p.Mp + j] = st.d;
          p.ps[vt * p.Mp + j] = st.s;
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
// SPLIT (the FP32-input form): dZ leaves as two BF16 planes, hi = bf16(x) at
// dz and lo = bf16(x - hi) at dz + plane, so hi + lo carries x to about 16
// significant bits; both planes of 128 tokens fill the stage one plane of
// 256 tokens fills, so the tile is staged and stored in two halves.
template <bool ENT, bool SPLIT = false>
struct EpiDzT {
  struct Params {
    uint16_t* dz;
    int64_t ldz, c0, vc_valid;
    const float* stats;
    const int64_t* targets;
    const float* grad_output;
    const int32_t* n_valid;
    const float* entropy;       // ENT: the forward's entropy
    const float* grad_entropy;  // ENT: adds grad_entropy[m] dH/dz
    float eps;
    int reduce_loss;
    int64_t ignore_idx, M, V;
    int64_t v0, Vg;  // W holds vocabulary rows v0 .. v0 + V - 1 of Vg (0, V unless sharded)
    float scale;     // logits are scale times the accumulators (1 unscaled)
    float slog2e;    // fl(scale log2(e))
    int64_t plane;   // SPLIT: elements from the hi plane to the lo plane
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t* smem) {
    // every per-token input of the lane's four tokens first, so that they
    // share one memory round trip
    int64_t tg[NB];
    f32x4_t sv[NB];
    float go[NB], gh[NB], hv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      const bool in = j < p.M;
      tg[b] = in ? p.targets[j] : p.ignore_idx;
      sv[b] = in ? *reinterpret_cast<const f32x4_t*>(p.stats + 4 * j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      go[b] = (in && !p.reduce_loss) ? p.grad_output[j] : 0.0f;
      gh[b] = (ENT && in) ? p.grad_entropy[j] : 0.0f;
      hv[b] = (ENT && in) ? p.entropy[j] : 0.0f;
    }
    float gscale = 0.0f;
    if (p.reduce_loss) {
      const int32_t nv = p.n_valid[0];
      gscale = p.grad_output[0] / (float)(nv > 0 ? nv : 1);
    }
    const int64_t vrow0 = i0 + wr * 128 + 4 * (lane >> 5);  // chunk-local row of r = 0
    // a wave whose 128 rows all lie in the chunk skips the per-element test
    const bool full = p.vc_valid - (i0 + wr * 128) >= 128;
    const int64_t lim64 = p.vc_valid - vrow0;
    const int lim = lim64 > 128 ? 128 : (lim64 < 0 ? 0 : (int)lim64);

    // Terms of token column b.  Rows that give zero (ignored token, padding
    // column) or NaN (target out of range) are folded into the arithmetic:
    // g = 0 or NaN, and an exponent pushed to -inf so that exp() is 0 for
    // every finite logit.
    // lse2 = fl(lse log2(e)) is the exponent's offset; its rounding, lo =
    // lse log2(e) - lse2, is taken back out of the factors that multiply the
    // exponential (ge = 2^-lo g, gHe = 2^-lo gH), so the error of p does not
    // grow with |m| (up to |m| of about 2^29).
    struct Tok {
      int64_t t;
      float g, ge, lse2, gH, gHe, ez;
      bool live;
    };
    auto token = [&](int b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      Tok k{-1, 0.0f, 0.0f, 1e30f, 0.0f, 0.0f, 0.0f, false};
      if (j < p.M) {
        k.t = tg[b];
        if (k.t != p.ignore_idx) {
          if (k.t >= 0 && k.t < p.Vg) {
            k.live = true;
            // the gradient with respect to the accumulators: scale times the
            // one with respect to the logits
            k.g = p.scale * (p.reduce_loss ? gscale : go[b]);
            const float ld = log2_hw(sv[b][1]);
            k.lse2 = __builtin_fmaf(sv[b][0], kLog2e, ld);
            const float lo = __builtin_fmaf(sv[b][0], kLog2e, -k.lse2) + ld;
            // 2^-lo = 1 - lo ln 2 to within (lo ln 2)^2 / 2 for |lo| < 2^-10
            float f = __builtin_fmaf(-lo, kLn2, 1.0f);
            if (!(fabsf(lo) < 0x1p-10f)) f = exp2_hw(-lo);
            k.ge = k.g * f;
            if (ENT) {  // dH/dz_v = p_v (E_p[z] - z_v), E_p[z] = lse - H
              k.gH = p.scale * gh[b];
              k.gHe = k.gH * f;
              k.ez = k.lse2 * kLn2 - hv[b];
            }
          } else {
            k.g = __builtin_nanf("");
            k.ge = k.g;
          }
        }
      }
      return k;
    };
    auto value = [&](const Tok& k, float goff, float z) {
      const float ex = exp2_hw(__builtin_fmaf(z, p.slog2e, -k.lse2));
      return ENT ? ex * __builtin_fmaf(k.gHe, __builtin_fmaf(-p.scale, z, k.ez), k.ge) - goff
                 : ex * k.ge - goff;
    };
    // The target's element also gets -(1 - eps) g: only a lane whose target
    // lies in this wave's rows (rarely any) recomputes that one value.
    auto target_row = [&](const Tok& k) {
      const int64_t tr64 = k.t - p.v0 - p.c0 - vrow0;
      return (k.live && tr64 >= 0 && tr64 < 128 && ((tr64 >> 2) & 1) == 0 && tr64 < lim)
                 ? (int)tr64
                 : -1;
    };

    // Straight from the accumulators to memory, no LDS round trip: lanes l
    // and l + 32 hold rows 8 q + [0, 4) and 8 q + [4, 8) of block a for the
    // same token, so one v_permlane32_swap per dword pair gives lane l rows
    // [0, 8) and [16, 24) of the block and lane l + 32 rows [8, 16) and
    // [24, 32): two 16-byte stores per lane and block (per plane), 32
    // consecutive bytes of a token row from each lane pair.
    const int64_t row0 = i0 + wr * 128 + 8 * (lane >> 5);  // chunk of r = 0 after the swap
    auto swap_store = [&](uint32_t (&w)[8], uint16_t* dst) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto sw = __builtin_amdgcn_permlane32_swap(w[4 * h + d], w[4 * h + 2 + d], false,
                                                           false);
          w[4 * h + d] = sw[0];
          w[4 * h + 2 + d] = sw[1];
        }
      *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
    };
    // the per-element row test only where the wave's rows run past the
    // chunk (a uniform branch: a select per element there, none elsewhere)
    auto columns = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
  #pragma unroll
      for (int b = 0; b < NB; ++b) {
        const Tok k = token(b);
        const float goff = k.g * (p.eps / (float)p.Vg);
        const int tl = target_row(k);
        uint16_t* const drow = p.dz + (j0 + wc * WN + b * 32 + (lane & 31)) * p.ldz + row0;
  #pragma unroll
        for (int a = 0; a < NA; ++a) {
          float val[16];
  #pragma unroll
          for (int q = 0; q < 4; ++q)
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = value(k, goff, acc[a][b][4 * q + e]);
              val[4 * q + e] = (!MASKED || a * 32 + 8 * q + e < lim) ? x : 0.0f;
            }
          // the target's element (rarely in this block): the same value less
          // (1 - eps) g
          if (tl >= 0 && (tl >> 5) == a) {
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              if (tl == a * 32 + 8 * (r >> 2) + (r & 3))
                val[r] = value(k, goff, acc[a][b][r]) - k.g * (1.0f - p.eps);
          }
          uint32_t w[8];
  #pragma unroll
          for (int r = 0; r < 8; ++r) w[r] = pack_bf16x2(val[2 * r], val[2 * r + 1]);
          if constexpr (SPLIT) {
            // the lo plane: what the BF16 hi value leaves of each FP32 value
            uint32_t wl[8];
  #pragma unroll
            for (int r = 0; r < 8; ++r)
              wl[r] = pack_bf16x2(val[2 * r] - bf16_lo(w[r]), val[2 * r + 1] - bf16_hi(w[r]));
            swap_store(wl, drow + p.plane + a * 32);
          }
          swap_store(w, drow + a * 32);
        }
      }
    };
    if (full)
      columns(std::false_type{});
    else
      columns(std::true_type{});
  }
};

// Backward dW of a chunk: rows = hidden (h), cols = vocabulary of the chunk.
struct EpiDw {
  struct Params {
    uint16_t* dW;
    int64_t H, c0, vc_valid;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
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
// dW of a chunk in FP32 (the FP32-input form): rows = hidden, cols = vocabulary.
struct EpiDwF32 {
  struct Params {
    float* dW;
    int64_t H, c0, vc_valid;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
                               int wr, int wc, int lane, uint16_t*) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t j = j0 + wc * WN + b * 32 + (lane & 31);
      if (j >= p.vc_valid) continue;
      float* row = p.dW + (p.c0 + j) * p.H;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t i = i0 + wr * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
          if (i < p.H)
            *reinterpret_cast<f32x4_t*>(row + i) =
                f32x4_t{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                        acc[a][b][4 * q + 3]};
        }
    }
  }
};

struct EpiDx {
  struct Params {
    float* accbuf;
    uint16_t* dX;
    int64_t H, M;
    int mode;
  };
  __device__ static void apply(const Params& p, f32x16_t (&acc)[NA][NB], int64_t i0, int64_t j0,
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
  float* partial_w;  // shard mode with ENT: (M) entropy statistic w
};

// ENT: the partials carry the entropy accumulator too (and the entropy is written).
template <bool ENT>
__global__ __launch_bounds__(256) void lce_merge_kernel(MergeParams p) {
  using S = typename std::conditional<ENT, LseEntState, LseState>::type;
  __shared__ S sh[8][32];
  const int tl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + tl;
  S st;
  st.m = kNegInf;
  st.d = 0.0f;
  st.s = 0.0f;
  if constexpr (ENT) st.w = 0.0f;
  if (j < p.M) {
    // tiles in a fixed order (group grp takes every 8th); unrolled so that
    // the loads of several tiles are in flight at once
#pragma unroll 8
    for (int64_t vt = grp; vt < p.n_vt; vt += 8) {
      const int64_t o = vt * p.Mp + j;
      S q;
      q.m = p.pm[o];
      q.d = p.pd[o];
      q.s = p.ps[o];
      if constexpr (ENT) q.w = p.pw[o];
      lse_merge(st, q);
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
    if constexpr (ENT) p.partial_w[j] = t != p.ignore_idx ? st.w : 0.0f;
    return;
  }
  if (t == p.ignore_idx) {
    p.loss_tok[j] = 0.0f;
    *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.entropy) p.entropy[j] = 0.0f;
    return;
  }
  if constexpr (ENT) p.entropy[j] = entropy_of(st.d, st.w);
  const bool t_ok = t >= 0 && t < p.V;
  const float zt = t_ok ? p.zt[j] : __builtin_nanf("");
  const float mean = st.s / (float)p.V;
  const float loss = ce_row_loss(st.m, st.d, zt, mean, p.eps);
  p.loss_tok[j] = t_ok ? loss : __builtin_nanf("");
  *reinterpret_cast<f32x4_t*>(p.stats + 4 * j) = f32x4_t{st.m, st.d, zt, mean};
}

// ---- host side ------------------------------------------------------------------

template <class Epi, bool PD, bool QD, int NSEG>
hipError_t run_gemm(const Segs<NSEG>& G, int64_t rows, int64_t cols, int64_t K,
                    const typename Epi::Params& ep, hipStream_t stream) {
  const int64_t n_ti = (rows + BM - 1) / BM, n_tj = (cols + BN - 1) / BN;
  const int64_t n = n_ti * n_tj;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX / 2) return hipErrorInvalidValue;
  // every operand has k_limit = K
  if (K % (2 * BK) != 0 || K == 0)
    hipLaunchKernelGGL((gemm_kernel<Epi, PD, QD, true, NSEG>), dim3((unsigned)n), dim3(NT), 0,
                       stream, G, K, (int)n_ti, (int)n_tj, ep);
  else
    hipLaunchKernelGGL((gemm_kernel<Epi, PD, QD, false, NSEG>), dim3((unsigned)n), dim3(NT), 0,
                       stream, G, K, (int)n_ti, (int)n_tj, ep);
  return hipGetLastError();
}

template <class Epi, bool PD, bool QD>
hipError_t run_gemm(const Operand& P, const Operand& Q, int64_t rows, int64_t cols, int64_t K,
                    const typename Epi::Params& ep, hipStream_t stream) {
  return run_gemm<Epi, PD, QD, 1>(Segs<1>{{P}, {Q}}, rows, cols, K, ep, stream);
}

inline bool needs_mask(int64_t K) { return K % (2 * BK) != 0 || K == 0; }

template <class EA, bool PA, bool QA, bool MA, class EB, bool PB, bool QB, bool MB, int NSEG>
hipError_t launch2(const GemmProblem<NSEG>& A, const typename EA::Params& ea,
                   const GemmProblem<NSEG>& B, const typename EB::Params& eb, int64_t n,
                   hipStream_t stream) {
  hipLaunchKernelGGL((gemm2_kernel<EA, PA, QA, MA, EB, PB, QB, MB, NSEG>), dim3((unsigned)n),
                     dim3(NT), 0, stream, A, ea, B, eb);
  return hipGetLastError();
}

// Problem A (rows x cols, K) and problem B in one launch, A's tiles first.
template <class EA, bool PA, bool QA, class EB, bool PB, bool QB, int NSEG>
hipError_t run_gemm2(const Segs<NSEG>& GA, int64_t rowsA, int64_t colsA, int64_t KA,
                     const typename EA::Params& ea, const Segs<NSEG>& GB, int64_t rowsB,
                     int64_t colsB, int64_t KB, const typename EB::Params& eb,
                     hipStream_t stream) {
  GemmProblem<NSEG> A{GA, KA, (int)((rowsA + BM - 1) / BM), (int)((colsA + BN - 1) / BN)};
  GemmProblem<NSEG> B{GB, KB, (int)((rowsB + BM - 1) / BM), (int)((colsB + BN - 1) / BN)};
  const int64_t n = (int64_t)A.n_ti * A.n_tj + (int64_t)B.n_ti * B.n_tj;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX / 2) return hipErrorInvalidValue;
  const bool ma = needs_mask(KA), mb = needs_mask(KB);
  if (!ma && !mb)
    return launch2<EA, PA, QA, false, EB, PB, QB, false, NSEG>(A, ea, B, eb, n, stream);
  if (!ma && mb)
    return launch2<EA, PA, QA, false, EB, PB, QB, true, NSEG>(A, ea, B, eb, n, stream);
  if (ma && !mb)
    return launch2<EA, PA, QA, true, EB, PB, QB, false, NSEG>(A, ea, B, eb, n, stream);
  return launch2<EA, PA, QA, true, EB, PB, QB, true, NSEG>(A, ea, B, eb, n, stream);
}

template <class EA, bool PA, bool QA, class EB, bool PB, bool QB, bool MB, class EC, bool PC,
          bool QC, bool MC, int NSEG>
hipError_t launch3(const GemmProblem<NSEG>& A, const typename EA::Params& ea,
                   const GemmProblem<NSEG>& B, const typename EB::Params& eb,
                   const GemmProblem<NSEG>& C, const typename EC::Params& ec, int64_t n,
                   hipStream_t stream) {
  hipLaunchKernelGGL((gemm3_kernel<EA, PA, QA, false, EB, PB, QB, MB, EC, PC, QC, MC, NSEG>),
                     dim3((unsigned)n), dim3(NT), 0, stream, A, ea, B, eb, C, ec);
  return hipGetLastError();
}

// Problems A, B and C in one launch, in that order.  A's K must need no mask
// (the callers pass a whole chunk); B's and C's may.
template <class EA, bool PA, bool QA, class EB, bool PB, bool QB, class EC, bool PC, bool QC,
          int NSEG>
hipError_t run_gemm3(const Segs<NSEG>& GA, int64_t rowsA, int64_t colsA, int64_t KA,
                     const typename EA::Params& ea, const Segs<NSEG>& GB, int64_t rowsB,
                     int64_t colsB, int64_t KB, const typename EB::Params& eb,
                     const Segs<NSEG>& GC, int64_t rowsC, int64_t colsC, int64_t KC,
                     const typename EC::Params& ec, hipStream_t stream) {
  GemmProblem<NSEG> A{GA, KA, (int)((rowsA + BM - 1) / BM), (int)((colsA + BN - 1) / BN)};
  GemmProblem<NSEG> B{GB, KB, (int)((rowsB + BM - 1) / BM), (int)((colsB + BN - 1) / BN)};
  GemmProblem<NSEG> C{GC, KC, (int)((rowsC + BM - 1) / BM), (int)((colsC + BN - 1) / BN)};
  const int64_t n = (int64_t)A.n_ti * A.n_tj + (int64_t)B.n_ti * B.n_tj + (int64_t)C.n_ti * C.n_tj;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX / 2 || needs_mask(KA)) return hipErrorInvalidValue;
  const bool mb = needs_mask(KB), mc = needs_mask(KC);
  if (!mb && !mc)
    return launch3<EA, PA, QA, EB, PB, QB, false, EC, PC, QC, false, NSEG>(A, ea, B, eb, C, ec, n,
                                                                          stream);
  if (!mb && mc)
    return launch3<EA, PA, QA, EB, PB, QB, false, EC, PC, QC, true, NSEG>(A, ea, B, eb, C, ec, n,
                                                                         stream);
  if (mb && !mc)
    return launch3<EA, PA, QA, EB, PB, QB, true, EC, PC, QC, false, NSEG>(A, ea, B, eb, C, ec, n,
                                                                         stream);
  return launch3<EA, PA, QA, EB, PB, QB, true, EC, PC, QC, true, NSEG>(A, ea, B, eb, C, ec, n,
                                                                      stream);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool lce_make_plan(int64_t M, int64_t H, int64_t V, LcePlan* plan, bool f32) {
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
  p.f32 = f32;
  // FP32 inputs: hi and lo planes of X, then of W
  p.xplane = f32 ? align256((size_t)M * H * 2) : 0;
  p.wplane = f32 ? align256((size_t)V * H * 2) : 0;
  p.off_xs = 0;
  p.off_ws = 2 * p.xplane;
  const size_t split = 2 * p.xplane + 2 * p.wplane;
  const size_t part = align256((size_t)p.n_vtiles * p.Mp * 4);
  const size_t fwd = split + 4 * part + align256((size_t)p.Mp * 4);
  // backward: dZ of one chunk (Mp x chunk, token-major; two planes with FP32
  // inputs) and the dX accumulator (BF16 output over several chunks only)
  const size_t dz = align256((size_t)p.Mp * p.chunk * 2);
  p.dzplane = f32 ? (int64_t)(dz / 2) : 0;
  const size_t dx = (!f32 && p.n_chunks > 1) ? align256((size_t)p.Mp * H * 4) : 0;
  // the BF16 form with several chunks keeps two dZ buffers: chunk c + 1's dZ
  // is formed in the launch that reads chunk c's
  const bool two_dz = !f32 && p.n_chunks > 1;
  p.off_part = split;
  p.off_dz = split;
  p.off_dz2 = two_dz ? split + dz : split;
  p.off_dx = split + (f32 || two_dz ? 2 : 1) * dz;
  const size_t bwd = p.off_dx + dx;
  p.fwd_bytes = fwd;
  p.total = fwd > bwd ? fwd : bwd;
  *plan = p;
  return true;
}

namespace {

// hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest even; x - hi is
// exact in FP32, so hi + lo carries x to about 16 significant bits (the
// FP32-input form runs its GEMMs on these planes: x y ~ xh yh + xh yl + xl yh).
// n4 groups of four elements; every thread takes up to four groups, a grid
// stride apart, with their loads in flight together.
__global__ __launch_bounds__(256) void split_bf16_kernel(const f32x4_t* in, u32x2_t* hi,
                                                         u32x2_t* lo, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < n4; i0 += 4 * stride) {
    f32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = i < n4 ? __builtin_nontemporal_load(in + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= n4) break;
      const uint32_t h01 = pack_bf16x2(v[u][0], v[u][1]), h23 = pack_bf16x2(v[u][2], v[u][3]);
      hi[i] = u32x2_t{h01, h23};
      lo[i] = u32x2_t{pack_bf16x2(v[u][0] - bf16_lo(h01), v[u][1] - bf16_hi(h01)),
                      pack_bf16x2(v[u][2] - bf16_lo(h23), v[u][3] - bf16_hi(h23))};
    }
  }
}

// Split n FP32 elements (n a multiple of 4) into planes hi and lo.
hipError_t run_split(const float* in, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t want = (n4 + 4 * 256 - 1) / (4 * 256);
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(split_bf16_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4_t*>(in), reinterpret_cast<u32x2_t*>(hi),
                     reinterpret_cast<u32x2_t*>(lo), n4);
  return hipGetLastError();
}

}  // namespace

namespace {

// The BF16 planes of FP32 inputs in the workspace, filled from X and W.
struct SplitOps {
  const uint16_t *Xh, *Xl, *Wh, *Wl;
};

SplitOps split_inputs(const LcePlan& plan, const void* X, const void* W, char* ws,
                      hipStream_t stream, hipError_t* err) {
  uint16_t* xh = reinterpret_cast<uint16_t*>(ws + plan.off_xs);
  uint16_t* xl = reinterpret_cast<uint16_t*>(ws + plan.off_xs + plan.xplane);
  uint16_t* wh = reinterpret_cast<uint16_t*>(ws + plan.off_ws);
  uint16_t* wl = reinterpret_cast<uint16_t*>(ws + plan.off_ws + plan.wplane);
  *err = run_split(static_cast<const float*>(X), xh, xl, plan.M * plan.H, stream);
  if (*err == hipSuccess)
    *err = run_split(static_cast<const float*>(W), wh, wl, plan.V * plan.H, stream);
  return SplitOps{xh, xl, wh, wl};
}

}  // namespace

hipError_t launch_lce_forward(const LcePlan& plan, const LceFwdArgs& a, hipStream_t stream) {
  const size_t part = align256((size_t)plan.n_vtiles * plan.Mp * 4);
  float* pm = reinterpret_cast<float*>(a.ws + plan.off_part);
  float* pd = reinterpret_cast<float*>(a.ws + plan.off_part + part);
  float* ps = reinterpret_cast<float*>(a.ws + plan.off_part + 2 * part);
  float* pw = reinterpret_cast<float*>(a.ws + plan.off_part + 3 * part);
  float* zt = reinterpret_cast<float*>(a.ws + plan.off_part + 4 * part);
  hipError_t e;
  // the entropy accumulator: for the entropy output, or a shard's entropy statistic
  const bool ent = a.entropy != nullptr || a.partial_w != nullptr;
  const EpiLseT<true>::Params ept{pm, pd, ps, pw, zt, a.targets, plan.M, plan.V, plan.Mp,
                                  a.ignore_idx, a.v0, a.scale, a.scale * kLog2e};
  const EpiLseT<false>::Params epf{pm, pd, ps, pw, zt, a.targets, plan.M, plan.V, plan.Mp,
                                   a.ignore_idx, a.v0, a.scale, a.scale * kLog2e};
  if (!plan.f32) {
    const uint16_t* X = static_cast<const uint16_t*>(a.X);
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    Operand P{W, plan.H, plan.V, plan.H};
    Operand Q{X, plan.H, plan.M, plan.H};
    e = ent
            ? run_gemm<EpiLseT<true>, false, false>(P, Q, plan.V, plan.Mp, plan.H, ept, stream)
            : run_gemm<EpiLseT<false>, false, false>(P, Q, plan.V, plan.Mp, plan.H, epf, stream);
  } else {
    // Z = Xh Wh^T + Xh Wl^T + Xl Wh^T, one tile summing the three products
    const SplitOps o = split_inputs(plan, a.X, a.W, a.ws, stream, &e);
    if (e != hipSuccess) return e;
    const Segs<3> G{{{o.Wh, plan.H, plan.V, plan.H},
                     {o.Wl, plan.H, plan.V, plan.H},
                     {o.Wh, plan.H, plan.V, plan.H}},
                    {{o.Xh, plan.H, plan.M, plan.H},
                     {o.Xh, plan.H, plan.M, plan.H},
                     {o.Xl, plan.H, plan.M, plan.H}}};
    e = ent
            ? run_gemm<EpiLseT<true>, false, false, 3>(G, plan.V, plan.Mp, plan.H, ept, stream)
            : run_gemm<EpiLseT<false>, false, false, 3>(G, plan.V, plan.Mp, plan.H, epf, stream);
  }
  if (e != hipSuccess) return e;
  MergeParams mp{pm, pd, ps, pw, zt, a.targets, plan.M, plan.Mp, plan.V, plan.n_vtiles,
                 a.ignore_idx, a.eps, a.loss_tok, a.stats, a.entropy, a.v0, a.partial,
                 a.partial_w};
  if (ent)
    hipLaunchKernelGGL(lce_merge_kernel<true>, dim3((unsigned)((plan.M + 31) / 32)), dim3(256), 0,
                       stream, mp);
  else
    hipLaunchKernelGGL(lce_merge_kernel<false>, dim3((unsigned)((plan.M + 31) / 32)), dim3(256), 0,
                       stream, mp);
  return hipGetLastError();
}

// Zero n 16-byte words (dW of an empty batch).
__global__ __launch_bounds__(256) void lce_zero_kernel(u32x4_t* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = u32x4_t{0u, 0u, 0u, 0u};
}

namespace {

// The FP32-input backward: per vocabulary chunk, dZ in two BF16 planes from
// the three-product logits, then dX += dZ W_c and dW_c = dZ^T X each as one
// tile summing three products of the planes (dZh Wh + dZh Wl + dZl Wh, and
// likewise with X), FP32 outputs.
template <bool ENT>
hipError_t backward_f32(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream) {
  hipError_t e;
  const SplitOps o = split_inputs(plan, a.X, a.W, a.ws, stream, &e);
  if (e != hipSuccess) return e;
  uint16_t* dzh = reinterpret_cast<uint16_t*>(a.ws + plan.off_dz);
  const uint16_t* dzl = dzh + plan.dzplane;
  const int64_t H = plan.H, M = plan.M;
  for (int64_t c = 0; c < plan.n_chunks; ++c) {
    const int64_t c0 = c * plan.chunk;
    const int64_t vc = (plan.V - c0) < plan.chunk ? (plan.V - c0) : plan.chunk;
    const uint16_t* Whc = o.Wh + c0 * H;
    const uint16_t* Wlc = o.Wl + c0 * H;
    {
      const Segs<3> G{{{Whc, H, vc, H}, {Wlc, H, vc, H}, {Whc, H, vc, H}},
                      {{o.Xh, H, M, H}, {o.Xh, H, M, H}, {o.Xl, H, M, H}}};
      typename EpiDzT<ENT, true>::Params ep{dzh, plan.ldz, c0, vc, a.stats, a.targets,
                                            a.grad_output, a.n_valid, a.entropy, a.grad_entropy,
                                            a.eps, a.reduce_loss, a.ignore_idx, M, plan.V,
                                            a.v0, a.Vg, a.scale, a.scale * kLog2e,
                                            plan.dzplane};
      e = run_gemm<EpiDzT<ENT, true>, false, false, 3>(G, vc, plan.Mp, H, ep, stream);
      if (e != hipSuccess) return e;
    }
    {
      const Segs<3> GX{{{Whc, H, H, vc}, {Wlc, H, H, vc}, {Whc, H, H, vc}},
                       {{dzh, plan.ldz, M, vc}, {dzh, plan.ldz, M, vc}, {dzl, plan.ldz, M, vc}}};
      EpiDx::Params ex{static_cast<float*>(a.dX), nullptr, H, M, c > 0 ? 1 : 0};
      const Segs<3> GW{{{o.Xh, H, H, M}, {o.Xl, H, H, M}, {o.Xh, H, H, M}},
                       {{dzh, plan.ldz, vc, M}, {dzh, plan.ldz, vc, M}, {dzl, plan.ldz, vc, M}}};
      EpiDwF32::Params ew{static_cast<float*>(a.dW), H, c0, vc};
      e = run_gemm2<EpiDx, true, false, EpiDwF32, true, true, 3>(GX, H, M, vc, ex, GW, H, vc, M,
                                                                 ew, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// The BF16 backward, per vocabulary chunk c: dZ_c (vocabulary x tokens, K = H,
// both operands K-contiguous) into one of two buffers; then dX += dZ_c W_c
// (hidden x tokens, K = the chunk's vocabulary: W_c read dim-contiguous, dZ
// K-contiguous) and the chunk's dW rows (hidden x vocabulary, K = tokens: X
// and dZ both read dim-contiguous) in one launch, dX's longer tiles first, and
// with them dZ_{c+1} into the other buffer, its short tiles last.
template <bool ENT>
hipError_t backward_bf16(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream) {
  uint16_t* const dzb[2] = {reinterpret_cast<uint16_t*>(a.ws + plan.off_dz),
                            reinterpret_cast<uint16_t*>(a.ws + plan.off_dz2)};
  float* dxacc = reinterpret_cast<float*>(a.ws + plan.off_dx);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const int64_t H = plan.H, M = plan.M;
  auto rows_of = [&](int64_t c) {
    const int64_t c0 = c * plan.chunk;
    return (plan.V - c0) < plan.chunk ? (plan.V - c0) : plan.chunk;
  };
  auto dz_problem = [&](int64_t c, uint16_t* dz, Segs<1>* G, typename EpiDzT<ENT>::Params* ep) {
    const int64_t c0 = c * plan.chunk, vc = rows_of(c);
    *G = Segs<1>{{Operand{W + c0 * H, H, vc, H}}, {Operand{X, H, M, H}}};
    *ep = typename EpiDzT<ENT>::Params{dz, plan.ldz, c0, vc, a.stats, a.targets, a.grad_output,
                                       a.n_valid, ENT ? a.entropy : nullptr,
                                       ENT ? a.grad_entropy : nullptr, a.eps, a.reduce_loss,
                                       a.ignore_idx, M, plan.V, a.v0, a.Vg, a.scale,
                                       a.scale * kLog2e};
  };
  hipError_t e;
  {
    Segs<1> G;
    typename EpiDzT<ENT>::Params ep;
    dz_problem(0, dzb[0], &G, &ep);
    e = run_gemm<EpiDzT<ENT>, false, false, 1>(G, rows_of(0), plan.Mp, H, ep, stream);
    if (e != hipSuccess) return e;
  }
  for (int64_t c = 0; c < plan.n_chunks; ++c) {
    const int64_t c0 = c * plan.chunk, vc = rows_of(c);
    uint16_t* dz = dzb[c & 1];
    const Segs<1> GX{{Operand{W + c0 * H, H, H, vc}}, {Operand{dz, plan.ldz, M, vc}}};
    const int mode = (c > 0 ? 1 : 0) | (c + 1 == plan.n_chunks ? 2 : 0);
    const EpiDx::Params ex{dxacc, static_cast<uint16_t*>(a.dX), H, M, mode};
    const Segs<1> GW{{Operand{X, H, H, M}}, {Operand{dz, plan.ldz, vc, M}}};
    const EpiDw::Params ew{static_cast<uint16_t*>(a.dW), H, c0, vc};
    if (c + 1 < plan.n_chunks && plan.off_dz2 != plan.off_dz && !needs_mask(vc)) {
      Segs<1> GZ;
      typename EpiDzT<ENT>::Params ez;
      dz_problem(c + 1, dzb[(c + 1) & 1], &GZ, &ez);
      e = run_gemm3<EpiDx, true, false, EpiDw, true, true, EpiDzT<ENT>, false, false, 1>(
          GX, H, M, vc, ex, GW, H, vc, M, ew, GZ, rows_of(c + 1), plan.Mp, H, ez, stream);
      if (e != hipSuccess) return e;
    } else {
      e = run_gemm2<EpiDx, true, false, EpiDw, true, true, 1>(GX, H, M, vc, ex, GW, H, vc, M, ew,
                                                              stream);
      if (e != hipSuccess) return e;
      if (c + 1 < plan.n_chunks) {  // one dZ buffer: the next chunk's dZ after this launch
        Segs<1> GZ;
        typename EpiDzT<ENT>::Params ez;
        dz_problem(c + 1, dzb[(c + 1) & 1], &GZ, &ez);
        e = run_gemm<EpiDzT<ENT>, false, false, 1>(GZ, rows_of(c + 1), plan.Mp, H, ez, stream);
        if (e != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_lce_backward(const LcePlan& plan, const LceBwdArgs& a, hipStream_t stream) {
  if (plan.M == 0) {  // no token: dW = 0 (H is a multiple of 8, dW 16-byte aligned)
    const int64_t n = plan.V * plan.H / (plan.f32 ? 4 : 8);
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(lce_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<u32x4_t*>(a.dW), n);
    return hipGetLastError();
  }
  if (plan.f32)
    return a.grad_entropy ? backward_f32<true>(plan, a, stream)
                          : backward_f32<false>(plan, a, stream);
  return a.grad_entropy ? backward_bf16<true>(plan, a, stream)
                        : backward_bf16<false>(plan, a, stream);
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
