// Logits cross-entropy kernels for gfx950: the statistics-saving forward row
// sweep, the deterministic mean, and the gradient-rebuilding backward sweep.
//
// What they compute follows the TransformerEngine cross-entropy API page
// (Description: fused online-softmax, FP32 math for BF16/FP32 input; I/O
// Contract) and the TransformerEngine PR that saves statistics instead of the
// derivative (Changes; Sequence Diagram: one forward kernel on a single GPU,
// backward rebuilds the gradient from input, targets, stats and grad_output).
//
// Design for CDNA4: one workgroup per row (512 threads in the forward, 1024
// in the backward); every lane streams 16-byte vectors (8 BF16 or 4 FP32)
// with four loads in flight before any arithmetic, the row's last partial
// chunk included (masked, not one vector at a time); one exponential per
// logit (the running max is updated once per 4-vector chunk, not per
// element); the row state is merged across the wavefront with butterfly
// shuffles and across wavefronts in LDS.  The workgroup sizes were measured
// on MI355X (see kFwdThreads).
#include <type_traits>

#include "vce_device.h"
#include "vce_internal.h"

namespace vce {

#define LDS_AS __attribute__((address_space(3)))

namespace {

// Threads per row: the forward reads each element once and reduces the row,
// the backward reads and writes it.  Measured on MI355X: at 4096 rows of
// 32000 BF16 the forward takes 46-48 us with 512 threads and 58-61 us with
// 1024 (more rows in flight per CU, shorter reductions), and the same at
// 128256 columns, while rows of at most 48 KB are read faster by 256 (4096
// rows of 8000 BF16: 17.7 against 24.2 us; of 16032: 25.5 against 30 us; of
// 24000: 34.6 against 40 us; at 32000, 44.8 against 44.0 us); the backward is
// fastest with 1024 (85 vs 89 us at 32000,
// 364 vs 397 us at 128256) on rows over 32 KB, and with 512 on shorter ones,
// where 1024 threads leave most lanes one vector or none (4096 rows of 8000
// BF16: 22.5 against 35.7 us; of 16032: 45.5-46.8 against 47.0-48.0 us;
// 256 threads are slower still at 16032).
constexpr int kFwdThreads = 512;
constexpr int kFwdThreadsShort = 256;
constexpr int64_t kFwdShortRowBytes = 49152;
constexpr int kBwdThreads = 1024;
constexpr int kBwdThreadsShort = 512;
constexpr int64_t kBwdShortRowBytes = 32768;
constexpr int kFbVecs = 32;  // most 16-byte vectors per thread the one-pass kernel holds
constexpr int kUnroll = 4;
// The forward's exponent offset is fl(m log2(e)) for the chunk's running
// maximum m, its rounding rho taken back out by a factor 2^-rho; |rho| grows
// to 2^6 at |m| = 2^30, the clamp below.  A chunk whose running maximum lies
// beyond it (a thread whose logits so far are all masked with a finite value
// such as -FLT_MAX) gets the offset of the clamped value instead, so its
// terms underflow to 0 or stay finite and vanish in the later merge with a
// larger maximum, which rescales them by e^(m_old - m_new) = 0, instead of
// turning d into inf or NaN.  A row whose final maximum itself exceeds 2^30
// in magnitude is outside this form.
constexpr float kFoldMaxM = 0x1p30f;

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // FP32
  using T = float;
  static constexpr int kVec = 4;
  __device__ static float load(const float* p) { return *p; }
};
template <>
struct Elem<1> {  // BF16
  using T = uint16_t;
  static constexpr int kVec = 8;
  __device__ static float load(const uint16_t* p) { return from_bf16(*p); }
};

// Row geometry: elements [0, head) and [tail0, V) are handled one by one, the
// 16-byte aligned body [head, tail0) as vectors.
struct RowSplit {
  int64_t head, nvec, tail0;
};

template <int DT>
__device__ __forceinline__ RowSplit split_row(const void* row, int64_t V) {
  constexpr int es = sizeof(typename Elem<DT>::T);
  constexpr int vec = Elem<DT>::kVec;
  uintptr_t a = reinterpret_cast<uintptr_t>(row);
  int64_t head = (int64_t)(((16u - (a & 15u)) & 15u) / es);
  if (head > V) head = V;
  RowSplit s;
  s.head = head;
  s.nvec = (V - head) / vec;
  s.tail0 = head + s.nvec * vec;
  return s;
}

// Values of one 16-byte vector as floats.
template <int DT>
__device__ __forceinline__ void unpack(const u32x4_t& w, float* z);
template <>
__device__ __forceinline__ void unpack<0>(const u32x4_t& w, float* z) {
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = __uint_as_float(w[i]);
}
template <>
__device__ __forceinline__ void unpack<1>(const u32x4_t& w, float* z) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[2 * i] = bf16_lo(w[i]);
    z[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <int DT>
__device__ __forceinline__ float vec_sum(const u32x4_t& w, const float* z, float acc);
template <>
__device__ __forceinline__ float vec_sum<0>(const u32x4_t&, const float* z, float acc) {
  return acc + ((z[0] + z[1]) + (z[2] + z[3]));
}
template <>
__device__ __forceinline__ float vec_sum<1>(const u32x4_t& w, const float*, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = bf16_pair_sum(w[i], acc);
  return acc;
}

// Fold n vectors (already loaded) into the running state; only the first
// `nvalid` take part (the others may hold anything).  S = LseEntState also
// accumulates w = sum exp(z - m) (z - m) log2(e) for the entropy.
template <int DT, int N, class S>
__device__ __forceinline__ void fold(S& st, const u32x4_t* w, int nvalid = N) {
  constexpr int vec = Elem<DT>::kVec;
  constexpr bool kEnt = __is_same(S, LseEntState);
  float z[N][vec];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    unpack<DT>(w[u], z[u]);
    if (u >= nvalid) {
#pragma unroll
      for (int i = 0; i < vec; ++i) z[u][i] = kNegInf;
    }
  }
  float cm = z[0][0];
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int i = 0; i < vec; ++i) cm = fmaxf(cm, z[u][i]);
  const float m_new = fmaxf(st.m, cm);
  const float mref = (m_new == kNegInf) ? 0.0f : m_new;
  // (z - m) log2(e) as z log2(e) - mL with mL = fl(m log2(e)): one FMA per
  // logit.  Every term of the chunk then carries the factor 2^rho of the
  // rounding rho = m log2(e) - mL (exact by an FMA), taken back out of the
  // chunk's sum below; what remains per term is the rounding of the FMA,
  // relative to (z - m) log2(e), so the terms near the maximum, which make
  // up d, are the most accurate.  A NaN logit makes d NaN.  The offset is
  // taken from m clamped to kFoldMaxM (see there).
  const float mc = fminf(fmaxf(mref, -kFoldMaxM), kFoldMaxM);
  const float mL = mc * kLog2e;
  const float rho = __builtin_fmaf(mc, kLog2e, -mL);
  float dpart[N], wpart[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    float acc = 0.0f, accw = 0.0f;
#pragma unroll
    for (int i = 0; i < vec; ++i) {
      const float t = __builtin_fmaf(z[u][i], kLog2e, -mL);
      const float e = exp2_hw(t);
      acc += e;
      // -inf logits: e = 0 and t = -inf; the clamp keeps 0 * t finite
      if constexpr (kEnt) accw = __builtin_fmaf(e, fmaxf(t, -200.0f), accw);
    }
    dpart[u] = acc;
    wpart[u] = accw;
  }
  float dsum = dpart[0];
#pragma unroll
  for (int u = 1; u < N; ++u) dsum += dpart[u];
  // 2^-rho = 1 - rho ln 2 to within (rho ln 2)^2 / 2: |rho| is half an FP32 ulp
  // of m log2(e) at most, below 2^-10 for |m| < 2^13; beyond, the exponential
  const float corr = fabsf(rho) < 0x1p-10f ? -rho * kLn2 : exp2_hw(-rho) - 1.0f;
  dsum = __builtin_fmaf(dsum, corr, dsum);
  const float f = exp_diff(st.m - mref);
  if constexpr (kEnt) {
    float wsum = wpart[0];
#pragma unroll
    for (int u = 1; u < N; ++u) wsum += wpart[u];
    // move the old w from the old max to the new one (nothing when empty)
    const float wold = st.d > 0.0f ? f * __builtin_fmaf((st.m - mref) * kLog2e, st.d, st.w) : 0.0f;
    st.w = wold + wsum;
  }
  st.d = __builtin_fmaf(st.d, f, dsum);
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (u < nvalid) st.s = vec_sum<DT>(w[u], z[u], st.s);
  st.m = m_new;
}

// fold() for a chunk of N vectors without the unpacked copy of the chunk:
// the same arithmetic in the same order (bitwise the same state), with each
// logit unpacked again where it is used instead of being held in registers
// between the chunk's max and its sum of exponentials (the one-pass kernel
// keeps the whole row in VGPRs and cannot spare 8 N more).
template <int DT, int N>
__device__ __forceinline__ void fold_lean(LseState& st, u32x4_t* w, int nvalid = N) {
  constexpr int vec = Elem<DT>::kVec;
  auto elem = [&](int u, int i) -> float {
    float z[vec];
    unpack<DT>(w[u], z);
    return u < nvalid ? z[i] : kNegInf;
  };
  float cm = elem(0, 0);
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int i = 0; i < vec; ++i) cm = fmaxf(cm, elem(u, i));
  // the unpacked values are not kept for the sums below
#pragma unroll
  for (int u = 0; u < N; ++u) asm volatile("" : "+v"(w[u]));
  const float m_new = fmaxf(st.m, cm);
  const float mref = (m_new == kNegInf) ? 0.0f : m_new;
  const float mc = fminf(fmaxf(mref, -kFoldMaxM), kFoldMaxM);
  const float mL = mc * kLog2e;
  const float rho = __builtin_fmaf(mc, kLog2e, -mL);
  float dsum = 0.0f;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < vec; ++i) acc += exp2_hw(__builtin_fmaf(elem(u, i), kLog2e, -mL));
    dsum = u == 0 ? acc : dsum + acc;
  }
  const float corr = fabsf(rho) < 0x1p-10f ? -rho * kLn2 : exp2_hw(-rho) - 1.0f;
  dsum = __builtin_fmaf(dsum, corr, dsum);
  const float f = exp_diff(st.m - mref);
  st.d = __builtin_fmaf(st.d, f, dsum);
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (u < nvalid) {
      float z[vec];
      unpack<DT>(w[u], z);
      st.s = vec_sum<DT>(w[u], z, st.s);
    }
  st.m = m_new;
}

template <int NW, class S>
__device__ __forceinline__ S block_reduce(S st, S* sh) {
  lse_wave_reduce(st);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = st;
  __syncthreads();
  S r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) lse_merge(r, sh[w]);
  return r;
}

template <bool ENT>
struct StateOf {
  using T = LseState;
};
template <>
struct StateOf<true> {
  using T = LseEntState;
};

// ENT: also the entropy of softmax(z) per row (0 for ignored rows).
// SHARD: the row holds vocabulary columns v0 .. v0 + V - 1 of a larger
// vocabulary; instead of the loss, write the shard's partial statistics
// (m, d, sum z, z_t if this shard holds the target else 0) for a later merge.
template <int DT, bool ENT, bool SHARD, int NT>
__global__ __launch_bounds__(NT) void ce_fwd_kernel(CeFwdParams p) {
  using T = typename Elem<DT>::T;
  using S = typename StateOf<ENT>::T;
  __shared__ S sh[NT / 64];
  const int64_t r = blockIdx.x;
  const int64_t i0 = r / p.d1, i1 = r - i0 * p.d1;
  const int64_t t = p.targets[i0 * p.ts0 + i1 * p.ts1];
  const int tid = threadIdx.x;
  if (t == p.ignore_idx) {
    if (tid == 0) {
      if (SHARD) {
        *reinterpret_cast<f32x4_t*>(p.partial + 4 * r) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (ENT) p.partial_w[r] = 0.0f;
      } else {
        p.loss_tok[r] = 0.0f;
        *reinterpret_cast<f32x4_t*>(p.stats + 4 * r) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (ENT) p.entropy[r] = 0.0f;
      }
    }
    return;
  }
  const int64_t V = p.V;
  const T* row = static_cast<const T*>(p.logits) + i0 * p.ls0 + i1 * p.ls1;
  const int64_t tl = t - p.v0;  // target column within this row
  const bool t_ok = (tl >= 0 && tl < V);
  float zt = SHARD ? 0.0f : __builtin_nanf("");
  if (tid == 0 && t_ok) zt = Elem<DT>::load(row + tl);

  const RowSplit rs = split_row<DT>(row, V);
  S st;
  st.m = kNegInf;
  st.d = 0.0f;
  st.s = 0.0f;
  if constexpr (ENT) st.w = 0.0f;  // one element: z - m = 0
  {
    const int64_t nscal = rs.head + (V - rs.tail0);
    if (tid < nscal) {
      const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
      const float z = Elem<DT>::load(row + idx);
      st.m = z;
      st.d = (z == kNegInf) ? 0.0f : 1.0f;
      st.s = z;
    }
  }
  const u32x4_t* vrow = reinterpret_cast<const u32x4_t*>(row + rs.head);
  int64_t j = tid;
  for (; j + (kUnroll - 1) * NT < rs.nvec; j += kUnroll * NT) {
    u32x4_t w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = __builtin_nontemporal_load(vrow + j + u * NT);
    fold<DT, kUnroll>(st, w);
  }
  if (j < rs.nvec) {  // last partial chunk: all its loads in flight together
    const int nvalid = (int)((rs.nvec - j + NT - 1) / NT);
    u32x4_t w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      w[u] = u < nvalid ? __builtin_nontemporal_load(vrow + j + u * NT)
                        : u32x4_t{0, 0, 0, 0};
    fold<DT, kUnroll>(st, w, nvalid);
  }
  const S tot = block_reduce<NT / 64>(st, sh);
  if (SHARD) {
    if (tid == 0) {
      *reinterpret_cast<f32x4_t*>(p.partial + 4 * r) = f32x4_t{tot.m, tot.d, tot.s, zt};
      if constexpr (ENT) p.partial_w[r] = tot.w;
    }
    return;
  }
  if (tid == 0) {
    if constexpr (ENT) p.entropy[r] = entropy_of(tot.d, tot.w);
    const float mean = tot.s / (float)V;
    const float loss = ce_row_loss(tot.m, tot.d, zt, mean, p.eps);
    p.loss_tok[r] = t_ok ? loss : __builtin_nanf("");
    *reinterpret_cast<f32x4_t*>(p.stats + 4 * r) = f32x4_t{tot.m, tot.d, zt, mean};
  }
}

// Averaged loss over non-ignored rows and their count, one workgroup, fixed
// summation order (bitwise reproducible): thread i sums rows i, i + 1024, ...
// in FP64 (the loss is read whatever the target, so both loads of a row go
// out together; an ignored row adds 0), then a butterfly over each
// wavefront's lanes (every lane ends with the same bits) and the sixteen
// wavefront sums in order.
__global__ __launch_bounds__(1024) void ce_mean_kernel(CeMeanParams p) {
  __shared__ double ssum[16];
  __shared__ int64_t scnt[16];
  double sum = 0.0;
  int64_t cnt = 0;
#pragma unroll 4
  for (int64_t r = threadIdx.x; r < p.N; r += 1024) {
    const int64_t i0 = r / p.d1, i1 = r - i0 * p.d1;
    const bool valid = p.targets[i0 * p.ts0 + i1 * p.ts1] != p.ignore_idx;
    const double l = p.loss_tok ? (double)p.loss_tok[r] : 0.0;
    sum += valid ? l : 0.0;
    cnt += valid ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off, 64);
    cnt += __shfl_xor(cnt, off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    ssum[wave] = sum;
    scnt[wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = ssum[0];
    int64_t c = scnt[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) {
      s += ssum[w];
      c += scnt[w];
    }
    if (p.loss_mean) p.loss_mean[0] = (float)(s / (double)(c > 0 ? c : 1));
    if (p.n_valid) p.n_valid[0] = (int32_t)c;
  }
}

template <int DT>
__device__ __forceinline__ void store_vec(void* dst, const float* g);
template <>
__device__ __forceinline__ void store_vec<0>(void* dst, const float* g) {
  u32x4_t w = {__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
               __float_as_uint(g[3])};
  __builtin_nontemporal_store(w, static_cast<u32x4_t*>(dst));
}
template <>
__device__ __forceinline__ void store_vec<1>(void* dst, const float* g) {
  u32x4_t w = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
               pack_bf16x2(g[6], g[7])};
  __builtin_nontemporal_store(w, static_cast<u32x4_t*>(dst));
}

template <int DT>
__device__ __forceinline__ void store_one(typename Elem<DT>::T* dst, float g);
template <>
__device__ __forceinline__ void store_one<0>(float* dst, float g) { *dst = g; }
template <>
__device__ __forceinline__ void store_one<1>(uint16_t* dst, float g) { *dst = to_bf16(g); }

// ENT: adds grad_entropy[r] dH/dz_v = grad_entropy[r] p_v (E_p[z] - z_v), with
// E_p[z] = lse - H from the forward's entropy.  W: the fewest waves per SIMD
// the register budget must allow (8 lets two 1024-thread workgroups share a
// CU, which pays off only for rows of 32..64 KB, measured).
template <int DT, bool ENT, int NT, int W = 1>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(W)))
void ce_bwd_kernel(CeBwdParams p) {
  using T = typename Elem<DT>::T;
  constexpr int vec = Elem<DT>::kVec;
  // workgroup (r, s): part s of p.splits of row r's vectors
  const int64_t r = blockIdx.x / p.splits;
  const int split = (int)(blockIdx.x - r * p.splits);
  const int64_t i0 = r / p.d1, i1 = r - i0 * p.d1;
  const int64_t t = p.targets[i0 * p.ts0 + i1 * p.ts1];
  const int tid = threadIdx.x;
  const int64_t V = p.V;
  const int64_t off = i0 * p.ls0 + i1 * p.ls1;
  const T* row = static_cast<const T*>(p.logits) + off;
  T* grow = static_cast<T*>(p.grad) + off;
  const RowSplit rs = split_row<DT>(grow, V);
  u32x4_t* gvec = reinterpret_cast<u32x4_t*>(grow + rs.head);
  const int64_t per = (rs.nvec + p.splits - 1) / p.splits;
  const int64_t jb = split * per, je = jb + per < rs.nvec ? jb + per : rs.nvec;

  // targets index the full vocabulary of Vg columns; this row holds columns
  // v0 .. v0 + V - 1 of it (v0 = 0, Vg = V unless sharded)
  if (t == p.ignore_idx || !(t >= 0 && t < p.Vg)) {
    // Ignored row: zero gradient.  Target out of range: NaN gradient.
    const float fill = (t == p.ignore_idx) ? 0.0f : __builtin_nanf("");
    float f[vec];
#pragma unroll
    for (int i = 0; i < vec; ++i) f[i] = fill;
    const int64_t nscal = rs.head + (V - rs.tail0);
    if (split == 0 && tid < nscal) {
      const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
      store_one<DT>(grow + idx, fill);
    }
    for (int64_t j = jb + tid; j < je; j += NT) store_vec<DT>(gvec + j, f);
    return;
  }

  float g;
  if (p.reduce_loss) {
    const int32_t nv = p.n_valid[0];
    g = p.grad_output[0] / (float)(nv > 0 ? nv : 1);
  } else {
    g = p.grad_output[r];
  }
  const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(p.stats + 4 * r);
  const float m = sv[0], d = sv[1];
  const float mref = (m == kNegInf) ? 0.0f : m;
  const float gs = g / d;
  const float goff = g * (p.eps / (float)p.Vg);
  const int64_t tl = t - p.v0;  // target column within this row (may lie outside)
  const float gt = g * (1.0f - p.eps);
  float gHd = 0.0f, ez = 0.0f;
  if constexpr (ENT) {
    gHd = p.grad_entropy[r] / d;
    ez = mref + kLn2 * log2_hw(d) - p.entropy[r];  // E_p[z] = lse - H
  }
  // Gradient of one logit, before the target correction: e^(z - m) from the
  // exact difference (its error does not grow with |z| or |m|, so elements
  // where p and the smoothing term nearly cancel keep their BF16 rounding).
  // A row with a finite mean logit holds no infinite or NaN logit, and with
  // |m| <= 2^100 no z - m can overflow, so it skips the clamp that -inf
  // logits (p = 0) need; the entropy term always clamps, so that
  // p (E_p[z] - z) stays 0 there.  A NaN logit has made d NaN in the
  // forward, hence the whole row.
  const bool finite_row = !ENT && __builtin_isfinite(sv[3]) && fabsf(m) <= 0x1p100f;
  auto sweep = [&](auto clamp) {
    auto gval = [&](float z) -> float {
      const float e = decltype(clamp)::value ? exp_diff(z - mref) : exp_diff_finite(z - mref);
      if constexpr (ENT)
        return e * __builtin_fmaf(gHd, ez - fmaxf(z, -1e30f), gs) - goff;
      else
        return e * gs - goff;
    };
    {
      const int64_t nscal = rs.head + (V - rs.tail0);
      if (split == 0 && tid < nscal) {
        const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
        const float z = Elem<DT>::load(row + idx);
        float gv = gval(z);
        if (idx == tl) gv -= gt;
        store_one<DT>(grow + idx, gv);
      }
    }
    // The logits row and the gradient row share their alignment within 16
    // bytes only if their base offsets agree; the host guarantees it (same
    // strides and equal base alignment), so the same split serves both.
    const u32x4_t* vrow = reinterpret_cast<const u32x4_t*>(row + rs.head);
    const int64_t tv = tl - rs.head;  // target position inside the vector body
    int64_t j = jb + tid;
    for (; j + (kUnroll - 1) * NT < je; j += kUnroll * NT) {
      u32x4_t w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) w[u] = __builtin_nontemporal_load(vrow + j + u * NT);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float z[vec];
        unpack<DT>(w[u], z);
        float gv[vec];
#pragma unroll
        for (int i = 0; i < vec; ++i) gv[i] = gval(z[i]);
        const int64_t base = (j + u * NT) * vec;
        if (tv >= base && tv < base + vec) {
#pragma unroll
          for (int i = 0; i < vec; ++i)
            if (base + i == tv) gv[i] -= gt;
        }
        store_vec<DT>(gvec + j + u * NT, gv);
      }
    }
    if (j < je) {  // last partial chunk: all its loads in flight together
      const int nvalid = (int)((je - j + NT - 1) / NT);
      u32x4_t w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (u < nvalid) w[u] = __builtin_nontemporal_load(vrow + j + u * NT);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (u >= nvalid) break;
        float z[vec];
        unpack<DT>(w[u], z);
        float gv[vec];
#pragma unroll
        for (int i = 0; i < vec; ++i) gv[i] = gval(z[i]);
        const int64_t base = (j + u * NT) * vec;
        if (tv >= base && tv < base + vec) {
#pragma unroll
          for (int i = 0; i < vec; ++i)
            if (base + i == tv) gv[i] -= gt;
        }
        store_vec<DT>(gvec + j + u * NT, gv);
      }
    }
  };
  if (finite_row)
    sweep(std::false_type{});
  else
    sweep(std::true_type{});
}

}  // namespace

// Forward and backward of one row in one pass, for a caller that knows
// grad_output when it asks for the loss (a terminal loss): the row is read
// once into registers (NV 16-byte vectors per thread, at most 512 x 32 x 16 B
// = 256 KB), its statistics are reduced exactly as ce_fwd_kernel reduces them
// (same threads, same chunks of four vectors, same order), loss and stats are
// written as ce_fwd_kernel writes them, and the gradient is written from the
// registers exactly as ce_bwd_kernel computes it from those statistics: one
// read and one write of the logits instead of two reads and one write.
template <int DT, int NV, int NT>
__global__ __launch_bounds__(NT) void ce_fb_kernel(CeFwdParams f, CeBwdParams b) {
  using T = typename Elem<DT>::T;
  constexpr int vec = Elem<DT>::kVec;
  constexpr int NC = NV / kUnroll;  // chunks of four vectors per thread
  __shared__ LseState sh[NT / 64];
  const int64_t r = blockIdx.x;
  const int64_t i0 = r / f.d1, i1 = r - i0 * f.d1;
  const int tid = threadIdx.x;
  const int64_t V = f.V;
  const int64_t off = i0 * f.ls0 + i1 * f.ls1;
  const T* row = static_cast<const T*>(f.logits) + off;
  T* grow = static_cast<T*>(b.grad) + off;
  const RowSplit rs = split_row<DT>(row, V);
  u32x4_t* gvec = reinterpret_cast<u32x4_t*>(grow + rs.head);
  const int64_t nscal = rs.head + (V - rs.tail0);
  // every load of this thread's share of the row goes out at once, before
  // the target is known (an ignored row drops them); vectors past the row
  // hold zeros
  const u32x4_t* vrow = reinterpret_cast<const u32x4_t*>(row + rs.head);
  u32x4_t w[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t j = tid + (int64_t)v * NT;
    w[v] = j < rs.nvec ? __builtin_nontemporal_load(vrow + j) : u32x4_t{0, 0, 0, 0};
  }
  const int64_t t = f.targets[i0 * f.ts0 + i1 * f.ts1];
  const bool t_ok = (t >= 0 && t < V);

  if (t == f.ignore_idx || !t_ok) {
    // ignored: loss 0, zero stats, zero gradient, the row is not read; a
    // target outside [0, V): the statistics as ce_fwd_kernel forms them,
    // NaN loss and a NaN gradient row
    const float fill = (t == f.ignore_idx) ? 0.0f : __builtin_nanf("");
    if (t != f.ignore_idx) {
      // statistics still come from the whole row (same order as the forward)
      LseState st{kNegInf, 0.0f, 0.0f};
      if (tid < nscal) {
        const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
        const float z = Elem<DT>::load(row + idx);
        st = LseState{z, (z == kNegInf) ? 0.0f : 1.0f, z};
      }
      int64_t j = tid;
      for (; j + (kUnroll - 1) * NT < rs.nvec; j += kUnroll * NT) {
        u32x4_t wc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) wc[u] = vrow[j + u * NT];
        fold<DT, kUnroll>(st, wc);
      }
      if (j < rs.nvec) {
        const int nvalid = (int)((rs.nvec - j + NT - 1) / NT);
        u32x4_t wc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          wc[u] = u < nvalid ? vrow[j + u * NT] : u32x4_t{0, 0, 0, 0};
        fold<DT, kUnroll>(st, wc, nvalid);
      }
      const LseState tot = block_reduce<NT / 64>(st, sh);
      if (tid == 0) {
        f.loss_tok[r] = __builtin_nanf("");
        *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) =
            f32x4_t{tot.m, tot.d, __builtin_nanf(""), tot.s / (float)V};
      }
      __syncthreads();  // every read of the row is done before it may be overwritten
    } else if (tid == 0) {
      f.loss_tok[r] = 0.0f;
      *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float fv[vec];
#pragma unroll
    for (int i = 0; i < vec; ++i) fv[i] = fill;
    if (tid < nscal) {
      const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
      store_one<DT>(grow + idx, fill);
    }
    for (int64_t j = tid; j < rs.nvec; j += NT) store_vec<DT>(gvec + j, fv);
    return;
  }

  // ---- forward: read the row into registers, reduce its statistics ----------
  float zt = __builtin_nanf("");
  if (tid == 0) zt = Elem<DT>::load(row + t);
  LseState st{kNegInf, 0.0f, 0.0f};
  float zs = 0.0f;  // this thread's scalar (head or tail) element, if any
  int64_t sidx = -1;
  if (tid < nscal) {
    sidx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
    zs = Elem<DT>::load(row + sidx);
    st = LseState{zs, (zs == kNegInf) ? 0.0f : 1.0f, zs};
  }
  // chunks of four vectors in the forward's order (its partial chunk folds
  // only its loaded vectors)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t j = tid + (int64_t)c * kUnroll * NT;
    if (j + (kUnroll - 1) * NT < rs.nvec) {
      fold<DT, kUnroll>(st, &w[c * kUnroll]);
    } else if (j < rs.nvec) {
      const int nvalid = (int)((rs.nvec - j + NT - 1) / NT);
      fold<DT, kUnroll>(st, &w[c * kUnroll], nvalid);
    }
  }
  const LseState tot = block_reduce<NT / 64>(st, sh);
  if (tid == 0) {
    const float mean = tot.s / (float)V;
    f.loss_tok[r] = ce_row_loss(tot.m, tot.d, zt, mean, f.eps);
    *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) = f32x4_t{tot.m, tot.d, zt, mean};
  }
  // every read of the row (the target logit included) is done before the
  // gradient may overwrite it
  __syncthreads();

  // ---- backward from the registers (the expressions of ce_bwd_kernel) --------
  float g;
  if (b.reduce_loss) {
    const int32_t nv = b.n_valid[0];
    g = b.grad_output[0] / (float)(nv > 0 ? nv : 1);
  } else {
    g = b.grad_output[r];
  }
  const float m = tot.m, d = tot.d;
  const float mref = (m == kNegInf) ? 0.0f : m;
  const float gs = g / d;
  const float goff = g * (b.eps / (float)V);
  const float gt = g * (1.0f - b.eps);
  // the clamp rule of ce_bwd_kernel, from the same statistics
  const bool finite_row = __builtin_isfinite(tot.s / (float)V) && fabsf(m) <= 0x1p100f;
  auto sweep = [&](auto clamp) {
    auto gval = [&](float z) -> float {
      const float e = decltype(clamp)::value ? exp_diff(z - mref) : exp_diff_finite(z - mref);
      return e * gs - goff;
    };
    if (sidx >= 0) {
      float gv = gval(zs);
      if (sidx == t) gv -= gt;
      store_one<DT>(grow + sidx, gv);
    }
    const int64_t tv = t - rs.head;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = tid + (int64_t)(c * kUnroll + u) * NT;
        if (j < rs.nvec) {
          float z[vec];
          unpack<DT>(w[c * kUnroll + u], z);
          float gv[vec];
#pragma unroll
          for (int i = 0; i < vec; ++i) gv[i] = gval(z[i]);
          const int64_t base = j * vec;
          if (tv >= base && tv < base + vec) {
#pragma unroll
            for (int i = 0; i < vec; ++i)
              if (base + i == tv) gv[i] -= gt;
          }
          store_vec<DT>(gvec + j, gv);
        }
      }
    }
  };
  if (finite_row)
    sweep(std::false_type{});
  else
    sweep(std::true_type{});
}

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Buffer descriptor of `bytes` bytes at p, built from wave-uniform scalars
// (the row is the workgroup's, but the compiler cannot always tell, and a
// descriptor it thinks divergent costs a loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// The same descriptor as four scalar words, for store16_nt.
__device__ __forceinline__ u32x4_t row_rsrc_words(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xffffu,
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// 16 bytes per lane to the buffer at voff + soff, non-temporal, then two wait
// states before anything may write the data registers.  Written out because
// the compiler puts no wait state behind a 16-byte buffer store with a scalar
// offset, and a data register written right after it lost a dword in some
// lanes (measured on gfx950: lanes 12..15 of each 16 kept the next value).
__device__ __forceinline__ void store16_nt(const u32x4_t& v, uint32_t voff, const u32x4_t& rs,
                                           int soff) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, %3 offen nt\n\ts_nop 1"
               :
               : "v"(v), "v"(voff), "s"(rs), "s"(soff)
               : "memory");
}

// One vector's gradient values packed as stored: FP32 bits, or BF16 pairs
// rounded to nearest even.
template <int DT>
__device__ __forceinline__ u32x4_t pack_vec(const float* g);
template <>
__device__ __forceinline__ u32x4_t pack_vec<0>(const float* g) {
  return u32x4_t{__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                 __float_as_uint(g[3])};
}
template <>
__device__ __forceinline__ u32x4_t pack_vec<1>(const float* g) {
  return u32x4_t{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                 pack_bf16x2(g[6], g[7])};
}

// The one-pass kernel for rows over 48 KB (BF16 rows of 24577 .. 131072
// logits): held in registers alone, 8, 16 or 32 vectors a lane take about
// 120, 165 or 250 VGPRs, so two or one workgroups fit per CU, and each CU
// alternates between reading a row and computing on it.  Here the first NR
// vectors of a thread's share stay in VGPRs and the rest (if any) go straight
// from memory into LDS (buffer_load ... lds, read back by the same thread),
// so a lane fits in W waves' share of the register file (8 vectors: 70 VGPRs,
// three workgroups per CU; 16 or 32: 128, two) and a workgroup in under 80 KB
// of LDS at 128256 logits (measured 0.449 -> 0.390 ms per headline step,
// 124-129 -> 116-120 us at 4096 rows of 32000): one workgroup's arithmetic
// overlaps another's memory traffic.  Loads and
// stores go through buffer descriptors that end at the row's vector body (a
// read past it gives 0, a write past it is dropped: on gfx950 the range check
// covers the scalar offset too, measured), so the vector index goes in the
// scalar offset and no per-vector bounds branches or addresses are needed.
// Same threads, chunks, order and expressions as ce_fb_kernel: bitwise the
// same outputs.
template <int DT, int NR, int NV, int NT, int W = NT / 128>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(W)))
void ce_fb_split_kernel(CeFwdParams f, CeBwdParams b) {
  using T = typename Elem<DT>::T;
  constexpr int vec = Elem<DT>::kVec;
  constexpr int NC = NV / kUnroll;
  constexpr uint32_t kNt = 2;  // cache policy of the row's loads and stores: non-temporal
  extern __shared__ u32x4_t lrow[];  // vector j >= NR NT of the row at lrow[j - NR NT]
  __shared__ LseState sh[NT / 64];
  const int64_t r = blockIdx.x;
  // the row's coordinates as scalars (the division runs on the vector unit)
  const int64_t i0 = uniform64(r / f.d1), i1 = r - i0 * f.d1;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t V = f.V;
  const int64_t off = uniform64(i0 * f.ls0 + i1 * f.ls1);
  const T* row = static_cast<const T*>(f.logits) + off;
  T* grow = static_cast<T*>(b.grad) + off;
  const RowSplit rs = split_row<DT>(row, V);
  const int64_t nscal = rs.head + (V - rs.tail0);
  const int nvec = (int)rs.nvec;
  const __amdgpu_buffer_rsrc_t src = row_rsrc(row + rs.head, nvec * 16);
  const uint32_t voff = (uint32_t)tid * 16;
  // every load of this thread's share goes out at once, before the target is
  // known (an ignored row drops them)
  u32x4_t w[NR];
#pragma unroll
  for (int v = 0; v < NR; ++v)
    w[v] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(src, voff, v * NT * 16, kNt));
#pragma unroll
  for (int v = NR; v < NV; ++v)
    if (v * NT + 64 * wave < nvec)  // the wave's 64 vectors start inside the row
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src, (void LDS_AS*)(lrow + (v - NR) * NT + 64 * wave), 16, voff, v * NT * 16, 0, kNt);
  // vector slot v of this thread: from the registers or from LDS, 0 past the row
  auto vec_at = [&](int v) -> u32x4_t {
    if (v < NR) return w[v];
    return tid + v * NT < nvec ? lrow[(v - NR) * NT + tid] : u32x4_t{0, 0, 0, 0};
  };
  const int64_t t = f.targets[i0 * f.ts0 + i1 * f.ts1];
  const bool t_ok = (t >= 0 && t < V);

  if (t == f.ignore_idx || !t_ok) {
    // the LDS writes of the loads above land before the workgroup may end
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const float fill = (t == f.ignore_idx) ? 0.0f : __builtin_nanf("");
    if (t != f.ignore_idx) {
      // statistics still come from the whole row (same order as the forward)
      LseState st{kNegInf, 0.0f, 0.0f};
      if (tid < nscal) {
        const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
        const float z = Elem<DT>::load(row + idx);
        st = LseState{z, (z == kNegInf) ? 0.0f : 1.0f, z};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int j = tid + c * kUnroll * NT;
        if (j >= nvec) break;
        u32x4_t wc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) wc[u] = vec_at(c * kUnroll + u);
        if (j + (kUnroll - 1) * NT < nvec)
          fold_lean<DT, kUnroll>(st, wc);
        else
          fold_lean<DT, kUnroll>(st, wc, (nvec - j + NT - 1) / NT);
      }
      const LseState tot = block_reduce<NT / 64>(st, sh);
      if (tid == 0) {
        f.loss_tok[r] = __builtin_nanf("");
        *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) =
            f32x4_t{tot.m, tot.d, __builtin_nanf(""), tot.s / (float)V};
      }
      __syncthreads();  // every read of the row is done before it may be overwritten
    } else if (tid == 0) {
      f.loss_tok[r] = 0.0f;
      *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float fv[vec];
#pragma unroll
    for (int i = 0; i < vec; ++i) fv[i] = fill;
    if (tid < nscal) {
      const int64_t idx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
      store_one<DT>(grow + idx, fill);
    }
    u32x4_t* gvec = reinterpret_cast<u32x4_t*>(grow + rs.head);
    for (int j = tid; j < nvec; j += NT) store_vec<DT>(gvec + j, fv);
    return;
  }

  // ---- forward: reduce the statistics (the chunks of ce_fwd_kernel) -------
  float zt = __builtin_nanf("");
  if (tid == 0) zt = Elem<DT>::load(row + t);
  LseState st{kNegInf, 0.0f, 0.0f};
  float zs = 0.0f;  // this thread's scalar (head or tail) element, if any
  int64_t sidx = -1;
  if (tid < nscal) {
    sidx = tid < rs.head ? tid : rs.tail0 + (tid - rs.head);
    zs = Elem<DT>::load(row + sidx);
    st = LseState{zs, (zs == kNegInf) ? 0.0f : 1.0f, zs};
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = tid + c * kUnroll * NT;
    if (j < nvec) {
      u32x4_t wc[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) wc[u] = vec_at(c * kUnroll + u);
      if (j + (kUnroll - 1) * NT < nvec)
        fold_lean<DT, kUnroll>(st, wc);
      else
        fold_lean<DT, kUnroll>(st, wc, (nvec - j + NT - 1) / NT);
    }
  }
  const LseState tot = block_reduce<NT / 64>(st, sh);
  if (tid == 0) {
    const float mean = tot.s / (float)V;
    f.loss_tok[r] = ce_row_loss(tot.m, tot.d, zt, mean, f.eps);
    *reinterpret_cast<f32x4_t*>(f.stats + 4 * r) = f32x4_t{tot.m, tot.d, zt, mean};
  }
  // every read of the row (the target logit included) is done before the
  // gradient may overwrite it
  __syncthreads();

  // ---- backward from registers and LDS (the expressions of ce_bwd_kernel) --
  float g;
  if (b.reduce_loss) {
    const int32_t nv = b.n_valid[0];
    g = b.grad_output[0] / (float)(nv > 0 ? nv : 1);
  } else {
    g = b.grad_output[r];
  }
  const float m = tot.m, d = tot.d;
  const float mref = (m == kNegInf) ? 0.0f : m;
  const float gs = g / d;
  const float goff = g * (b.eps / (float)V);
  const float gt = g * (1.0f - b.eps);
  const bool finite_row = __builtin_isfinite(tot.s / (float)V) && fabsf(m) <= 0x1p100f;
  const u32x4_t dst = row_rsrc_words(grow + rs.head, nvec * 16);
  auto sweep = [&](auto clamp) {
    auto gval = [&](float z) -> float {
      const float e = decltype(clamp)::value ? exp_diff(z - mref) : exp_diff_finite(z - mref);
      return e * gs - goff;
    };
    if (sidx >= 0) {
      float gv = gval(zs);
      if (sidx == t) gv -= gt;
      store_one<DT>(grow + sidx, gv);
    }
    const int64_t tv = t - rs.head;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int j = tid + v * NT;
      if (v >= NR && v * NT >= nvec) break;  // nothing of this slot or later is in the row
      float z[vec];
      unpack<DT>(vec_at(v), z);
      float gv[vec];
#pragma unroll
      for (int i = 0; i < vec; ++i) gv[i] = gval(z[i]);
      const int64_t base = (int64_t)j * vec;
      if (tv >= base && tv < base + vec) {
#pragma unroll
        for (int i = 0; i < vec; ++i)
          if (base + i == tv) gv[i] -= gt;
      }
      store16_nt(pack_vec<DT>(gv), voff, dst, v * NT * 16);
    }
  };
  if (finite_row)
    sweep(std::false_type{});
  else
    sweep(std::true_type{});
}

// Per-row merge of vocabulary-shard statistics, shards in fixed order
// (bitwise reproducible): m = max m_k, d = sum d_k exp(m_k - m), sum z, and
// z_t from the shard holding the target (the others contribute 0); then the
// loss and the saved statistics as ce_fwd_kernel writes them, with the mean
// logit and eps / V over the full vocabulary.
template <bool ENT>
__global__ __launch_bounds__(256) void ce_merge_shards_kernel(CeMergeParams p) {
  using S = typename StateOf<ENT>::T;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= p.N) return;
  const int64_t i0 = r / p.d1, i1 = r - i0 * p.d1;
  const int64_t t = p.targets[i0 * p.ts0 + i1 * p.ts1];
  if (t == p.ignore_idx) {
    p.loss_tok[r] = 0.0f;
    *reinterpret_cast<f32x4_t*>(p.stats + 4 * r) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (ENT) p.entropy[r] = 0.0f;
    return;
  }
  S st;
  st.m = kNegInf;
  st.d = 0.0f;
  st.s = 0.0f;
  if constexpr (ENT) st.w = 0.0f;
  float zt = 0.0f;
  for (int64_t k = 0; k < p.n_shards; ++k) {
    const f32x4_t q = *reinterpret_cast<const f32x4_t*>(p.partials + (k * p.N + r) * 4);
    S b;
    b.m = q[0];
    b.d = q[1];
    b.s = q[2];
    if constexpr (ENT) b.w = p.partials_w[k * p.N + r];
    lse_merge(st, b);
    zt += q[3];
  }
  const bool t_ok = t >= 0 && t < p.V;
  if (!t_ok) zt = __builtin_nanf("");
  const float mean = st.s / (float)p.V;
  const float loss = ce_row_loss(st.m, st.d, zt, mean, p.eps);
  p.loss_tok[r] = t_ok ? loss : __builtin_nanf("");
  *reinterpret_cast<f32x4_t*>(p.stats + 4 * r) = f32x4_t{st.m, st.d, zt, mean};
  if constexpr (ENT) p.entropy[r] = entropy_of(st.d, st.w);
}

// Causal label shift: out[r] = the target one position later along the
// sequence axis (axis 0 or 1 of the (d0, d1) grid), ignore_idx at the last
// position.  out is (d0, d1) contiguous in flattened row order.
__global__ __launch_bounds__(256) void shift_targets_kernel(ShiftParams p) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= p.N) return;
  const int64_t i0 = r / p.d1, i1 = r - i0 * p.d1;
  const int64_t j0 = p.seq_axis == 0 ? i0 + 1 : i0;
  const int64_t j1 = p.seq_axis == 1 ? i1 + 1 : i1;
  const bool last = (p.seq_axis == 0) ? (j0 >= p.d0) : (j1 >= p.d1);
  p.out[r] = last ? p.ignore_idx : p.targets[j0 * p.ts0 + j1 * p.ts1];
}

hipError_t launch_shift_targets(const ShiftParams& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(shift_targets_kernel, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

// Rows of at most kFwdShortRowBytes take the smaller workgroup (the one-pass
// kernel follows the same rule, so that its statistics are reduced in the
// same order).
static inline bool fwd_short_row(int dtype, int64_t V) {
  return V * (dtype == 0 ? 4 : 2) <= kFwdShortRowBytes;
}

template <int DT, bool ENT, bool SHARD>
void launch_fwd(const CeFwdParams& p, int64_t N, hipStream_t stream) {
  if (fwd_short_row(DT, p.V))
    hipLaunchKernelGGL((ce_fwd_kernel<DT, ENT, SHARD, kFwdThreadsShort>), dim3((unsigned)N),
                       dim3(kFwdThreadsShort), 0, stream, p);
  else
    hipLaunchKernelGGL((ce_fwd_kernel<DT, ENT, SHARD, kFwdThreads>), dim3((unsigned)N),
                       dim3(kFwdThreads), 0, stream, p);
}

hipError_t launch_ce_forward(const CeFwdParams& p, int dtype, int64_t N, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (p.partial) {
    const bool ent = p.partial_w != nullptr;
    if (dtype == 0 && !ent)
      launch_fwd<0, false, true>(p, N, stream);
    else if (dtype == 0)
      launch_fwd<0, true, true>(p, N, stream);
    else if (!ent)
      launch_fwd<1, false, true>(p, N, stream);
    else
      launch_fwd<1, true, true>(p, N, stream);
    return hipGetLastError();
  }
  const bool ent = p.entropy != nullptr;
  if (dtype == 0 && !ent)
    launch_fwd<0, false, false>(p, N, stream);
  else if (dtype == 0)
    launch_fwd<0, true, false>(p, N, stream);
  else if (!ent)
    launch_fwd<1, false, false>(p, N, stream);
  else
    launch_fwd<1, true, false>(p, N, stream);
  return hipGetLastError();
}

hipError_t launch_ce_merge_shards(const CeMergeParams& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  const dim3 g((unsigned)((p.N + 255) / 256)), b(256);
  if (p.entropy)
    hipLaunchKernelGGL(ce_merge_shards_kernel<true>, g, b, 0, stream, p);
  else
    hipLaunchKernelGGL(ce_merge_shards_kernel<false>, g, b, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_ce_mean(const CeMeanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(ce_mean_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

namespace {

// Rows over 48 KB take ce_fb_split_kernel: up to 8 vectors a lane all in
// VGPRs at 6 waves per SIMD, up to 16 all in VGPRs at 4, beyond that
// kFbRegVecs in VGPRs and the rest in LDS, sized for the longest row of this
// V (no head elements); rows of at most 48 KB see launch_fb_dt.
constexpr int kFbRegVecs = 22;

template <int DT, int NR, int NV, int W = kFwdThreads / 128, int NT = kFwdThreads>
void launch_fb_split(const CeFwdParams& f, const CeBwdParams& b, dim3 g, int64_t nvec,
                     hipStream_t stream) {
  auto kern = ce_fb_split_kernel<DT, NR, NV, NT, W>;
  const int64_t in_lds = (nvec + 63) / 64 * 64 - (int64_t)NR * NT;
  const size_t lds = in_lds > 0 ? (size_t)in_lds * 16 : 0;
  // allow the dynamic LDS on whichever device the call runs (set per call: a
  // host-side attribute, no stream work, so graph capture is unaffected)
  if (lds > 0)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, g, dim3(NT), lds, stream, f, b);
}

template <int DT>
bool launch_fb_dt(const CeFwdParams& f, const CeBwdParams& b, int64_t N, hipStream_t stream) {
  // vectors per thread to hold the row (the 16-byte head/tail are scalars);
  // the workgroup size is the forward's for the same row
  const int64_t nvec = f.V / Elem<DT>::kVec;
  const dim3 g((unsigned)N);
  if (fwd_short_row(DT, f.V)) {
    // rows of at most 48 KB: 256 threads, as the forward; up to 8 vectors a
    // lane ce_fb_kernel (125 VGPRs, 4 workgroups per CU; the lean kernel at 6
    // waves per SIMD was 15% slower at 8000 BF16 columns), beyond that the
    // lean kernel at 4 waves (102 VGPRs where ce_fb_kernel took 173 and two
    // workgroups per CU: 24000 columns 94-98 -> 87 us)
    if (nvec <= 8 * kFwdThreadsShort)
      hipLaunchKernelGGL((ce_fb_kernel<DT, 8, kFwdThreadsShort>), g, dim3(kFwdThreadsShort), 0,
                         stream, f, b);
    else
      launch_fb_split<DT, 16, 16, 4, kFwdThreadsShort>(f, b, g, nvec, stream);
    return true;
  }
  if (nvec <= 8 * kFwdThreads)
    launch_fb_split<DT, 8, 8, 6>(f, b, g, nvec, stream);
  else if (nvec <= 16 * kFwdThreads)
    launch_fb_split<DT, 16, 16>(f, b, g, nvec, stream);
  else if (nvec <= kFbVecs * kFwdThreads)
    launch_fb_split<DT, kFbRegVecs, kFbVecs>(f, b, g, nvec, stream);
  else
    return false;
  return true;
}

}  // namespace

bool ce_fb_fits(int dtype, int64_t V) {
  return V / (dtype == 0 ? 4 : 8) <= (int64_t)kFbVecs * kFwdThreads;
}

hipError_t launch_ce_forward_backward(const CeFwdParams& f, const CeBwdParams& b, int dtype,
                                      int64_t N, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const bool ok = dtype == 0 ? launch_fb_dt<0>(f, b, N, stream) : launch_fb_dt<1>(f, b, N, stream);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// One workgroup per row; rows of at most kBwdShortRowBytes take the smaller
// workgroup.
// One workgroup per row, or per part of a long row: rows of at most
// kBwdShortRowBytes take the smaller workgroup; longer rows are cut into
// parts of about 8 vectors a lane (measured on 4096 rows of BF16: 128256
// columns in two parts 0.370 -> 0.355 ms, 65536 columns in two parts 0.5%
// faster, 32000 columns in two parts 30% slower, three parts of 128256 4%
// slower, four 8% slower).  Rows of 32..64 KB run two workgroups per CU:
// 32000 columns 1.5-3% faster in two A/B runs (90.2-93.2 -> 88.9-90.5 us);
// at 65536 columns it was 4% slower, at 16032 and 128256 no faster.
template <int DT, bool ENT>
void launch_bwd(const CeBwdParams& p0, int64_t N, hipStream_t stream) {
  CeBwdParams p = p0;
  if (p.V * (DT == 0 ? 4 : 2) <= kBwdShortRowBytes) {
    p.splits = 1;
    hipLaunchKernelGGL((ce_bwd_kernel<DT, ENT, kBwdThreadsShort>), dim3((unsigned)N),
                       dim3(kBwdThreadsShort), 0, stream, p);
  } else {
    constexpr int64_t part = 8 * kBwdThreads;  // vectors per part
    const int64_t nvec = p.V / Elem<DT>::kVec;
    int64_t splits = (nvec + part / 2) / part;
    if (splits < 1) splits = 1;
    if (N * splits > (int64_t)INT32_MAX) splits = 1;
    p.splits = (int)splits;
    const dim3 g((unsigned)(N * splits));
    if (p.V * (DT == 0 ? 4 : 2) <= 2 * kBwdShortRowBytes)
      hipLaunchKernelGGL((ce_bwd_kernel<DT, ENT, kBwdThreads, 8>), g, dim3(kBwdThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((ce_bwd_kernel<DT, ENT, kBwdThreads>), g, dim3(kBwdThreads), 0, stream,
                         p);
  }
}

hipError_t launch_ce_backward(const CeBwdParams& p, int dtype, int64_t N, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const bool ent = p.grad_entropy != nullptr;
  if (dtype == 0 && !ent)
    launch_bwd<0, false>(p, N, stream);
  else if (dtype == 0)
    launch_bwd<0, true>(p, N, stream);
  else if (!ent)
    launch_bwd<1, false>(p, N, stream);
  else
    launch_bwd<1, true>(p, N, stream);
  return hipGetLastError();
}

}  // namespace vce
