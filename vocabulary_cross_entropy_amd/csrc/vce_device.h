// Device helpers shared by the gfx950 kernels of libvce.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// ln 2 in two parts: kLn2Hi is ln 2 rounded to FP32, kLn2Lo the FP32 value
// nearest the remainder (ln 2 - kLn2Hi, about -1.9e-9).
constexpr float kLn2Hi = 0.693147182464599609375f;
constexpr float kLn2Lo = -1.9046542121259336e-09f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 2^x on the transcendental unit (v_exp_f32).  -inf gives 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// e^r for r <= 0 (r = z - m, a logit less its row maximum, formed exactly in
// FP32: for BF16 inputs and any FP32 pair within a factor of two the
// difference is exact).  t = fl(r log2 e) goes to the transcendental unit
// unchanged, and the rounding left in t is put back as the factor 1 + c with
// c = r - t ln 2, taken with ln 2 in two parts (the Cody-Waite reduction): the
// result carries the exponential unit's own error and about one FP32 rounding,
// independent of the size of z or m.  exp_diff_finite takes a finite r;
// exp_diff also takes -inf, giving 0 (the clamp keeps t finite: e^-256 is 0
// in FP32), and gives 0 for a NaN r too, so callers that must propagate NaN
// logits do so through the row statistics.
__device__ __forceinline__ float exp_diff_finite(float r) {
  const float t = r * kLog2e;
  float c = __builtin_fmaf(-t, kLn2Hi, r);
  c = __builtin_fmaf(-t, kLn2Lo, c);
  const float e0 = exp2_hw(t);
  return __builtin_fmaf(e0, c, e0);
}
__device__ __forceinline__ float exp_diff(float r) { return exp_diff_finite(fmaxf(r, -256.0f)); }

// Rescale factors of an online-softmax merge of two partial states with
// maxima am and bm: the side with the larger maximum keeps factor 1 (exactly
// exp_diff(0)), the other gets e^(m_small - m_big).  One exponential per
// merge; two empty sides (both -inf) give factors 1 and 0 on zero sums.
__device__ __forceinline__ void merge_factors(float am, float bm, float& fa, float& fb) {
  const bool a_big = am >= bm;
  const float f = exp_diff(a_big ? bm - am : am - bm);
  fa = a_big ? 1.0f : f;
  fb = a_big ? f : 1.0f;
}

// BF16 pair packed in one dword -> two floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum of the two BF16 values of a dword, added to acc (v_dot2_f32_bf16 with ones).
__device__ __forceinline__ float bf16_pair_sum(uint32_t w, float acc) {
  bf16x2_t x = __builtin_bit_cast(bf16x2_t, w);
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}

// Two floats -> BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float from_bf16(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Online log-sum-exp state: running max m, d = sum exp(z - m), s = sum z.
struct LseState {
  float m, d, s;
};

// Merge b into a.  Either side may be empty (m = -inf, d = 0).  The sums of
// products are written as explicit FMAs so that every kernel rounds them the
// same way (the compiler would otherwise pick which product to fuse).
__device__ __forceinline__ void lse_merge(LseState& a, const LseState& b) {
  const float m = fmaxf(a.m, b.m);
  float fa, fb;
  merge_factors(a.m, b.m, fa, fb);
  a.d = __builtin_fmaf(a.d, fa, b.d * fb);
  a.s = a.s + b.s;
  a.m = m;
}

// Butterfly reduction of an LseState over the 64 lanes of a wavefront.
__device__ __forceinline__ void lse_wave_reduce(LseState& st) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    LseState o;
    o.m = __shfl_xor(st.m, off, 64);
    o.d = __shfl_xor(st.d, off, 64);
    o.s = __shfl_xor(st.s, off, 64);
    lse_merge(st, o);
  }
}

// Online state with the entropy accumulator as well:
//   w = sum exp(z - m) (z - m) log2(e),
// so that the entropy of softmax(z) is H = ln(2) (log2(d) - w / d)
// (H = lse - E_p[z] = ln d - sum p (z - m)).  Terms stay bounded
// (exp(x) x >= -1/e for x <= 0), so no large sum cancels.
struct LseEntState {
  float m, d, s, w;
};

// Merge b into a: each side's w is moved from its own max to the common one,
// sum exp(z - m*) (z - m*) = f (w - (m* - m) log2(e) d) with f = exp(m - m*).
// An empty side (d = 0) contributes nothing.
__device__ __forceinline__ void lse_merge(LseEntState& a, const LseEntState& b) {
  const float m = fmaxf(a.m, b.m);
  const float mref = (m == kNegInf) ? 0.0f : m;
  float fa, fb;
  merge_factors(a.m, b.m, fa, fb);
  const float wa = a.d > 0.0f ? fa * __builtin_fmaf((a.m - mref) * kLog2e, a.d, a.w) : 0.0f;
  const float wb = b.d > 0.0f ? fb * __builtin_fmaf((b.m - mref) * kLog2e, b.d, b.w) : 0.0f;
  a.d = __builtin_fmaf(a.d, fa, b.d * fb);
  a.s = a.s + b.s;
  a.w = wa + wb;
  a.m = m;
}

__device__ __forceinline__ void lse_wave_reduce(LseEntState& st) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    LseEntState o;
    o.m = __shfl_xor(st.m, off, 64);
    o.d = __shfl_xor(st.d, off, 64);
    o.s = __shfl_xor(st.s, off, 64);
    o.w = __shfl_xor(st.w, off, 64);
    lse_merge(st, o);
  }
}

// Per-row loss from the row statistics, written with explicit FMAs so that
// every kernel that forms it rounds the same way:
//   (lse - m) - (1 - eps)(z_t - m) - eps (mean z - m),  lse - m = ln d.
// The smoothing term is skipped for eps = 0 (a -inf logit would give 0 * inf).
__device__ __forceinline__ float ce_row_loss(float m, float d, float zt, float mean, float eps) {
  const float lse_shift = log2_hw(d) * kLn2;
  float loss = __builtin_fmaf(eps - 1.0f, zt - m, lse_shift);
  if (eps != 0.0f) loss = __builtin_fmaf(-eps, mean - m, loss);
  return loss;
}

// Entropy from a final state (NaN when d = 0: no finite logit).
__device__ __forceinline__ float entropy_of(float d, float w) {
  return kLn2 * (log2_hw(d) - w / d);
}

}  // namespace vce
