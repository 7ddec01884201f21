// Online-softmax generalized JSD over logits rows, in three passes
// (Liger-Kernel PR #1352 "Fuse log-softmax into fused_linear_jsd kernel",
// Details):
//   pass 1  row statistics m and d (running max and denominator, Milakov &
//           Gimelshein's online normalizer) for student and teacher together;
//   pass 2  the per-row loss and the cross-column term dX_sum;
//   pass 3  dX, written over the student logits when the caller asks for it
//           in place.
// With bf16 logits and a weight gradient, pass 3 also writes dX transposed
// for the weight-gradient product and sums the loss terms itself (per row
// over its column block, merged in a fixed order afterwards), so pass 2
// computes dX_sum alone (and the forward KL, which needs none, skips it).
// Everything from the loaded logit onward is fp32 (PR #1352 Details: the cast
// happens at load). Exponentials are base 2 (PR #1352 Details, last bullet):
// with k = log2(e)/T, a row's statistics are m = max z (in logit units, so
// the maximum is exact) and d = sum 2^((z - m) k), and an element's log2
// probability is a = (z - m) k - log2 d. A row may be split into S slices,
// each a workgroup; the slices' partial statistics and sums are merged in a
// fixed order, so results are deterministic run to run.
//
// Per element, with Q = 2^a_s (student), P = 2^a_t (teacher) and
// D = ln P - ln Q = (a_t - a_s) ln 2:
//   generalized: r = ln(beta e^D + 1 - beta), for fp32 logits from mix_log
//                (full relative accuracy at every D and beta; bf16 logits:
//                the base-2 form described at gen_terms),
//                ln(P/M) = D - r, ln(Q/M) = -r,
//                l = beta P (D - r) - (1-beta) Q r,   g = -(1-beta) Q r,
//                dA = g - Q G with G = sum_v g (dX_sum); for fp32 logits
//                the gradient terms are taken relative to the student's most
//                probable element (RowShift), which leaves dA unchanged and
//                keeps it accurate where it is a small difference of large
//                terms
//   forward KL:  l = P D - P + Q,  dA = Q - P          (sum_v P = 1 exactly)
//   reverse KL:  l = P - Q - Q D,  G = sum_v l,  dA = -Q D - Q G
// and an exact tie gives l = g = 0 (PR #1374 "Fix TVD gradient at p == q"):
// P == Q for fp32 logits, by one predicate and one select per element; for
// bf16 logits equal log2 probabilities a_s == a_t (then P == Q too), where
// the generalized terms vanish by themselves (gen_terms) and the KL branches
// take the fp32 test.
// The KL terms carry "- P + Q" (which sums to zero over a row) so that each
// term is O(D^2) and non-negative: the plain P D terms are O(D) and cancel
// across the row, which turns the fp32 rounding of the row normalizers into a
// first-order error of the loss. Near D = 0 the terms come from their Taylor
// series; the generalized divergence needs no such care (its derivative with
// respect to a normalizer error is itself O(loss)).
//
// Transcendentals use the hardware instructions (v_exp_f32 = 2^x, v_log_f32 =
// log2, v_rcp_f32). expm1 below |x| = 1/2 is a degree-9 Taylor polynomial and
// log1p below |y| = 1/4 the atanh series, so both keep full relative accuracy
// as their argument goes to 0.
#include "elem_math.h"
#include "kernels.h"
#include "plan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace fljsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Per-element terms of the divergence; see the file comment. Inputs are the
// log2 probabilities a_s, a_t. Outputs: Q and P, the loss term l, the
// gradient term g (dA = g - Q G) and gacc, the term summed into G. bf16
// logits take the generalized branch from gen_terms instead.
template <int MODE>
__device__ inline void jsd_terms(float as, float at, float beta, float& Q, float& P, float& l,
                                 float& g, float& gacc, const BetaWeights* bw = nullptr) {
  Q = hw_exp2(as);
  P = hw_exp2(at);
  if (P == Q) {  // exact tie: no loss, no gradient term
    l = 0.f;
    g = 0.f;
    gacc = 0.f;
    return;
  }
  const float t = at - as;    // log2(P / Q)
  const float D = t * kLn2;   // ln(P / Q)
  if (MODE == kModeForwardKL) {
    l = fabsf(D) < 0.25f ? Q * kl_fwd_series(D) : P * D - (P - Q);
    g = -P;
    gacc = 0.f;  // dA = Q - P needs no row sum
  } else if (MODE == kModeReverseKL) {
    l = fabsf(D) < 0.25f ? Q * kl_rev_series(D) : (P - Q) - Q * D;
    g = -Q * D;
    gacc = l;    // G = KL(Q||P), the row loss
  } else {
    // r and D - r each from mix_log, which keeps full relative accuracy at
    // every D and beta (no D + log1p(...) form whose two terms cancel when r
    // is much smaller than D, as for small beta).
    const float r = mix_log(D, t, bw->r);
    const float dmr = -mix_log(-D, -t, bw->dmr);
    l = beta * P * dmr - (1.f - beta) * Q * r;
    g = -(1.f - beta) * Q * r;
    gacc = g;
  }
}

// The bf16 generalized term of G (both pass-2 kernels, so that G does not
// depend on which outputs were asked for): gsum += g with
// g = -(1 - beta) Q ln(beta 2^t + 1 - beta), t = a_t - a_s clamped at 64
// (beyond it Q < 2^-64 P and the term is below any G); a tie (equal
// log-probabilities, or a masked column) adds 0. One exponential and one log
// from r's definition: G only enters dA = g - Q G, where an absolute error of
// a few 1e-7 in r is far below what the bf16 logits' own rounding (2^-9 of
// each logit, over T) does, and these passes are VALU-bound. The explicit
// fmaf keeps the compiler from contracting differently in the two kernels.
__device__ inline float gsum_plain(float gsum, float as, float at, float Q, float beta, float cg) {
  const float u = fmaf(beta, hw_exp2(fminf(at - as, 64.f)), 1.f - beta);
  return fmaf(as == at ? 0.f : Q, hw_log2(u) * cg, gsum);
}

// bf16 logits, generalized branch: the terms of one element, shared by every
// pass that evaluates them (pass 2's loss, pass 3's dZ with or without the
// transposed copy, pass 3's loss), so that no result depends on which
// outputs were asked for. In base 2, with t = a_t - a_s = D / ln 2,
// r2 = r / ln 2 for r = ln(beta e^D + 1 - beta):
//  - below |D| = 1/16, r's Taylor series to degree 4 (r is the cumulant
//    generating function of a Bernoulli(beta) variable, so the coefficient of
//    D^n / n! is its n-th cumulant; truncation below 1.3e-7 relative there),
//    which keeps a small r accurate relative to itself;
//  - beyond, with e = 2^-|t| and L = log2 of two positive terms: for t < 0,
//    r2 = L = log2(beta e + 1 - beta) and dmr2 = t - L; for t > 0,
//    L = log2((1 - beta) e + beta), r2 = t + L and dmr2 = -L. Nothing
//    overflows, and the smaller of r2 and dmr2 on each side never comes from
//    a difference (with t large and beta near 1, t - r2 would leave
//    -log2 beta ~ 1e-3 to the rounding of t). The argument is written
//    1 - c (1 - e), c the weight on e's side, so that it is exactly 1 at
//    e = 1: beta + (1 - beta) is not 1 in fp32 for most beta, and that bias,
//    the same sign at every element, reached 1e-3 of near-uniform row losses.
// dmr2 = (D - r) / ln 2 (t - r2 below 1/16). A tie (t == 0, finite logits)
// takes the series branch and gives r2 = dmr2 = 0, so both terms vanish with
// no select; masked columns (-inf in both rows) give NaN and the callers
// leave them out.
// Outputs: dz = grad_scale (g - Q G) with g = -(1 - beta) Q r, from
// nG = -G grad_scale and cg = -(1 - beta) ln 2 grad_scale; and the loss
// term over ln 2, l2 = (beta P (D - r) - (1 - beta) Q r) / ln 2.
struct GenBeta {
  float beta, cb, c2, c3, c4, cg;
};
__device__ inline GenBeta gen_beta(float beta, float grad_scale) {
  const float v = beta * (1.f - beta);  // the Bernoulli variance
  return {beta,
          1.f - beta,
          v * (0.5f * kLn2),
          v * (1.f - 2.f * beta) * (kLn2 * kLn2 / 6.f),
          v * (1.f - 6.f * v) * (kLn2 * kLn2 * kLn2 / 24.f),
          -(1.f - beta) * kLn2 * grad_scale};
}
struct GenRow {
  float ms, ls, mt, lt, nG;
};
__device__ inline GenRow gen_row(const float4& L, float G, float grad_scale) {
  return {L.x, -L.y, L.z, -L.w, -G * grad_scale};
}
// a_s = (z_s - m_s) k - log2 d_s, one FMA after an exact subtraction (two
// bf16 values): an element at its row's maximum gets exactly -log2 d, and
// rows that differ by a constant shift give equal log2 probabilities.
__device__ inline float gen_as(float z, float k, const GenRow& rw) {
  return fmaf(z - rw.ms, k, rw.ls);
}
__device__ inline float gen_at(float z, float k, const GenRow& rw) {
  return fmaf(z - rw.mt, k, rw.lt);
}
constexpr float kGenSmallT = 0.0625f / kLn2;  // |D| = 1/16
__device__ inline void gen_terms(float as, float at, float nG, const GenBeta& c, float& dz,
                                 float& l2) {
  const float Q = hw_exp2(as), P = hw_exp2(at);
  const float t = at - as;
  const bool neg = t < 0.f;
  const float e = hw_exp2(-fabsf(t));
  const float L = hw_log2(fmaf(-(neg ? c.beta : c.cb), 1.f - e, 1.f));
  float p = fmaf(c.c4, t, c.c3);
  p = fmaf(p, t, c.c2);
  p = fmaf(p, t, c.beta);
  const float rs = p * t;
  // Both branches evaluated, then selected (no divergent branch per element).
  const bool small = fabsf(t) < kGenSmallT;
  const float r2 = small ? rs : (neg ? L : t + L);
  const float dmr2 = small ? t - rs : (neg ? t - L : -L);
  const float Qr = Q * r2;
  l2 = fmaf(c.beta * P, dmr2, -c.cb * Qr);
  dz = fmaf(Q, nG, c.cg * Qr);
}

// Row statistics from the S pass-1 partials, merged in slice order by one
// thread and broadcast through LDS: returns (m_s, log2 d_s, m_t, log2 d_t).
__device__ inline float4 row_log_norms(const JsdArgs& a, int64_t row) {
  __shared__ float4 sh_L;
  if (threadIdx.x == 0) {
    const float4* st = a.stats + row * a.S;
    float4 acc = st[0];
    for (int s = 1; s < a.S; ++s) {
      const float4 o = st[s];
      md_merge(acc.x, acc.y, o.x, o.y, a.k2);
      md_merge(acc.z, acc.w, o.z, o.w, a.k2);
    }
    sh_L = make_float4(acc.x, hw_log2(acc.y), acc.z, hw_log2(acc.w));
  }
  __syncthreads();
  return sh_L;
}

// The teacher logit at the student's maximum, carried beside the student's
// (max, denominator): of two partial results the one with the larger maximum
// wins, and at equal maxima the larger teacher logit, so the merge is
// commutative (butterfly partners agree) and the result does not depend on
// the merge order.
__device__ inline float ref_merge(float m, float z, float mo, float zo) {
  return m > mo ? z : (mo > m ? zo : fmaxf(z, zo));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void jsd_stats_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* zs = static_cast<const T*>(a.zs) + row * a.ld;
  const T* zt = static_cast<const T*>(a.zt) + row * a.ld;
  const float k = a.k2;
  // fp32 rows also track the teacher logit at the student's maximum.
  constexpr bool kRef = sizeof(T) == 4;
  float ms = -INFINITY, ds = 0.f, mt = -INFINITY, dt = 0.f, zr = -INFINITY;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
    if constexpr (kRef) {
      float mx = ys[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, ys[i]);
      float zx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) zx = ys[i] == mx ? fmaxf(zx, yt[i]) : zx;
      if (mx != -INFINITY) zr = ref_merge(ms, zr, mx, zx);
    }
    md_update8(ms, ds, ys, k);
    md_update8(mt, dt, yt, k);
  }
  if constexpr (kRef) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float mo = __shfl_xor(ms, o, 64);
      const float dof = __shfl_xor(ds, o, 64);
      const float zo = __shfl_xor(zr, o, 64);
      zr = ref_merge(ms, zr, mo, zo);
      md_merge(ms, ds, mo, dof, k);
    }
  } else {
    wave_md(ms, ds, k);
  }
  wave_md(mt, dt, k);
  __shared__ float4 sh[kWaves];
  __shared__ float sh_ref[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    sh[wave] = make_float4(ms, ds, mt, dt);
    sh_ref[wave] = zr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 acc = sh[0];
    float ref = sh_ref[0];
    for (int w = 1; w < kWaves; ++w) {
      ref = ref_merge(acc.x, ref, sh[w].x, sh_ref[w]);
      md_merge(acc.x, acc.y, sh[w].x, sh[w].y, k);
      md_merge(acc.z, acc.w, sh[w].z, sh[w].w, k);
    }
    a.stats[row * a.S + s] = acc;
    if (kRef && a.ref != nullptr) a.ref[row * a.S + s] = ref;
  }
}

// fp32 gradient terms relative to a reference element (the student's most
// probable one). With Q summing to one over the row, dA = g - Q G is
// unchanged when every r_v is replaced by rho_v = r_v - r_c for any row
// constant r_c, and r(D_v; beta) - r(D_c; beta) = ln(w e^x + 1 - w) with
// x = D_v - D_c and w the mixture weight at D_c (mix_weights). Taking the
// reference at the student's maximum gives x from logit differences alone
// (the normalizers cancel), x = 0 exactly at that element, and small rho
// wherever the element's log-ratio is close to the reference's: a row whose
// probable elements all have P << Q (the divergence near its maximum, the
// gradient a small difference of O(Q) terms) keeps full relative accuracy,
// which the plain r_v - sum Q r loses to cancellation. Reverse KL takes the
// same shift with rho = x (its g is -Q D). When the reference is not finite
// (a -inf teacher logit there), the plain terms are used (D_c = 0).
struct RowShift {
  float4 L;        // (m_s, log2 d_s, m_t, log2 d_t)
  float zr;        // teacher logit at the student's maximum
  MixWeights mw;   // weights at the reference (beta, 1 - beta when unshifted)
  float rc;        // r at the reference (0 when unshifted)
  bool shifted;
};

// Row statistics and the reference, merged over the S slices by one thread
// and broadcast through LDS.
__device__ inline RowShift row_shift(const JsdArgs& a, int64_t row, bool generalized) {
  __shared__ RowShift sh;
  if (threadIdx.x == 0) {
    const float4* st = a.stats + row * a.S;
    const float* rf = a.ref + row * a.S;
    float4 acc = st[0];
    float zr = rf[0];
    for (int s = 1; s < a.S; ++s) {
      const float4 o = st[s];
      zr = ref_merge(acc.x, zr, o.x, rf[s]);
      md_merge(acc.x, acc.y, o.x, o.y, a.k2);
      md_merge(acc.z, acc.w, o.z, o.w, a.k2);
    }
    RowShift r;
    r.L = make_float4(acc.x, hw_log2(acc.y), acc.z, hw_log2(acc.w));
    r.zr = zr;
    // D_c in base 2: a_t - a_s at the reference, where a_s = -log2 d_s.
    const float tc = (zr - r.L.z) * a.k2 - r.L.w + r.L.y;
    r.shifted = isfinite(tc);
    const MixWeights plain = mix_weights(0.f, a.beta);
    r.mw = (generalized && r.shifted) ? mix_weights(tc, a.beta) : plain;
    r.rc = (generalized && r.shifted) ? mix_log(tc * kLn2, tc, plain) : 0.f;
    sh = r;
  }
  __syncthreads();
  return sh;
}

// The shifted gradient term of one element (fp32 generalized and reverse KL):
// returns g' with dA = g' - Q G', G' the row sum of g'. t = a_t - a_s.
template <int MODE>
__device__ inline float shifted_g(const RowShift& rs, float ys, float yt, float t, float Q, float P,
                                  float k, float beta) {
  const float xt = rs.shifted ? ((yt - rs.zr) - (ys - rs.L.x)) * k : t;
  const float x = xt * kLn2;
  float rho;
  if constexpr (MODE == kModeReverseKL) {
    rho = x;
    return Q > 0.f ? -Q * rho : 0.f;
  } else {
    rho = mix_log(x, xt, rs.mw);
    // A tie (P == Q) has r = 0 exactly (PR #1374), i.e. rho = -r_c.
    rho = P == Q ? -rs.rc : rho;
    return Q > 0.f ? -(1.f - beta) * Q * rho : 0.f;
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void jsd_loss_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* zs = static_cast<const T*>(a.zs) + row * a.ld;
  const T* zt = static_cast<const T*>(a.zt) + row * a.ld;
  // fp32: the gradient terms relative to the student's most probable element
  // (RowShift), except for the forward KL, whose dA = Q - P has no row sum.
  constexpr bool kShift = sizeof(T) == 4 && MODE != kModeForwardKL;
  RowShift rs{};
  float4 L;
  if constexpr (kShift) {
    rs = row_shift(a, row, MODE == kModeGeneralized);
    L = rs.L;
  } else {
    L = row_log_norms(a, row);
  }
  const float k = a.k2;
  const BetaWeights bw = beta_weights(a.beta);
  const float cg = -(1.f - a.beta) * kLn2;
  // bf16 generalized: the terms of gen_terms (loss over ln 2, rescaled below)
  // and G from gsum_plain.
  constexpr bool kGen16 = sizeof(T) == 2 && MODE == kModeGeneralized;
  const GenBeta gb = gen_beta(a.beta, 0.f);
  const GenRow rw = gen_row(L, 0.f, 0.f);
  // fp32 forward KL also sums Q and P over the elements below the student's
  // maximum and counts the elements at it, for pass 3's peak rewrite.
  constexpr bool kPeak = sizeof(T) == 4 && MODE == kModeForwardKL;
  float lsum = 0.f, gsum = 0.f, qrest = 0.f, prest = 0.f, npeak = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
    // Columns past the row end load as -inf in both rows: Q = P = 0, an exact
    // tie, which adds exactly 0 to every sum of jsd_terms and gsum_plain
    // (gen_terms' loss term is NaN there and is masked).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kGen16) {
        const float as = gen_as(ys[i], k, rw), at = gen_at(yt[i], k, rw);
        float dz, l2;
        gen_terms(as, at, 0.f, gb, dz, l2);
        lsum += i < n ? l2 : 0.f;
        gsum = gsum_plain(gsum, as, at, hw_exp2(as), a.beta, cg);
        continue;
      }
      float Q, P, l, g, gacc;
      const float as = (ys[i] - L.x) * k - L.y, at = (yt[i] - L.z) * k - L.w;
      jsd_terms<MODE>(as, at, a.beta, Q, P, l, g, gacc, &bw);
      if constexpr (kShift) gacc = shifted_g<MODE>(rs, ys[i], yt[i], at - as, Q, P, k, a.beta);
      lsum += l;
      gsum += gacc;
      if constexpr (kPeak) {
        const bool rest = ys[i] < L.x;
        qrest += rest ? Q : 0.f;
        prest += rest ? P : 0.f;
        npeak += rest ? 0.f : 1.f;
      }
    }
  }
  if constexpr (kGen16) lsum *= kLn2;
  lsum = wave_sum(lsum);
  gsum = wave_sum(gsum);
  __shared__ float2 sh[kWaves];
  __shared__ float4 sh_pk[kWaves];
  const int wave = threadIdx.x / 64;
  if constexpr (kPeak) {
    qrest = wave_sum(qrest);
    prest = wave_sum(prest);
    npeak = wave_sum(npeak);
    if ((threadIdx.x & 63) == 0) sh_pk[wave] = make_float4(qrest, prest, 0.f, npeak);
  }
  if ((threadIdx.x & 63) == 0) sh[wave] = make_float2(lsum, gsum);
  __syncthreads();
  if (threadIdx.x == 0) {
    float2 acc = sh[0];
    for (int w = 1; w < kWaves; ++w) {
      acc.x += sh[w].x;
      acc.y += sh[w].y;
    }
    a.lg[row * a.S + s] = acc;
    if (kPeak && a.peak != nullptr) {
      float4 pk = sh_pk[0];
      for (int w = 1; w < kWaves; ++w) {
        pk.x += sh_pk[w].x;
        pk.y += sh_pk[w].y;
        pk.z += sh_pk[w].z;
        pk.w += sh_pk[w].w;
      }
      a.peak[row * a.S + s] = pk;
    }
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void jsd_grad_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const T* zs = static_cast<const T*>(a.zs) + row * a.ld;
  const T* zt = static_cast<const T*>(a.zt) + row * a.ld;
  T* gr = static_cast<T*>(a.grad) + row * a.ld;
  constexpr bool kShift = sizeof(T) == 4 && MODE != kModeForwardKL;
  RowShift rs{};
  float4 L;
  if constexpr (kShift) {
    rs = row_shift(a, row, MODE == kModeGeneralized);
    L = rs.L;
  } else {
    L = row_log_norms(a, row);
  }
  const float k = a.k2;
  const BetaWeights bw = beta_weights(a.beta);
  constexpr bool kPeak = sizeof(T) == 4 && MODE == kModeForwardKL;
  __shared__ float sh_G;
  __shared__ float4 sh_pk;
  if (threadIdx.x == 0) {
    const float2* lg = a.lg + row * a.S;
    float2 acc = lg[0];
    for (int j = 1; j < a.S; ++j) {
      acc.x += lg[j].x;
      acc.y += lg[j].y;
    }
    sh_G = acc.y;
    if (s == 0) a.row_loss[row] = acc.x * a.row_scale;
    if constexpr (kPeak) {
      float4 pk = make_float4(0.f, 0.f, 0.f, 0.f);  // n = 0: no rewrite
      if (a.peak != nullptr) {
        const float4* pp = a.peak + row * a.S;
        pk = pp[0];
        for (int j = 1; j < a.S; ++j) {
          pk.x += pp[j].x;
          pk.y += pp[j].y;
          pk.z += pp[j].z;
          pk.w += pp[j].w;
        }
      }
      sh_pk = pk;
    }
  }
  __syncthreads();
  const float G = sh_G;
  constexpr bool kGen16 = sizeof(T) == 2 && MODE == kModeGeneralized;
  const GenBeta gb = gen_beta(a.beta, a.grad_scale);
  const GenRow rw = gen_row(L, G, a.grad_scale);
  // Peak rewrite (fp32 forward KL): when the student's row has one dominant
  // element p with Q_p near 1, Q_p - P_p computed from the rounded Q_p and P_p
  // keeps only ~1e-7 / |Q_p - P_p| relative accuracy. Summing the other
  // elements instead (the Q and the P each sum to one), Q_p - P_p =
  // P_rest - Q_rest. The sums carry the normalizers' rounding as a relative
  // error, as Q_p and P_p do, so the rewrite is taken only where its terms are
  // the smaller ones: Q_rest + P_rest < 1 (below Q_p + P_p). With a tied
  // maximum no element dominates and the plain form stays. (The other
  // branches need no rewrite: with the shifted terms the peak's g' is 0.)
  const float4 pk = kPeak ? sh_pk : make_float4(0.f, 0.f, 0.f, 0.f);
  const bool rewrite = kPeak && pk.w == 1.f && pk.x + pk.y < 1.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8], out[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kGen16) {
        float l2;
        gen_terms(gen_as(ys[i], k, rw), gen_at(yt[i], k, rw), rw.nG, gb, out[i], l2);
        continue;
      }
      float Q, P, l, g, gacc;
      const float as = (ys[i] - L.x) * k - L.y, at = (yt[i] - L.z) * k - L.w;
      jsd_terms<MODE>(as, at, a.beta, Q, P, l, g, gacc, &bw);
      if constexpr (kShift) g = shifted_g<MODE>(rs, ys[i], yt[i], at - as, Q, P, k, a.beta);
      float dA = (MODE == kModeForwardKL) ? (Q - P) : (g - Q * G);
      if (rewrite && ys[i] == L.x) dA = pk.y - pk.x;
      out[i] = dA * a.grad_scale;
    }
    store8(gr, v, n, a.vec_ok, out);
  }
}

// Pass 1 from the logits GEMMs' per-N-tile partials: one wave per row merges
// the student's and the teacher's partials in tile order into the row's
// statistics, stored as slice 0 of the stats array (the other slices get the
// merge identity, so the loss passes read the layout they always read).
__global__ __launch_bounds__(256) void jsd_stats_merge_kernel(JsdArgs a, const float2* part_s,
                                                              const float2* part_t,
                                                              int64_t tiles) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const float k = a.k2;
  float ms = -INFINITY, ds = 0.f, mt = -INFINITY, dt = 0.f;
  for (int64_t j = lane; j < tiles; j += 64) {
    const float2 ps = part_s[row * tiles + j];
    const float2 pt = part_t[row * tiles + j];
    md_merge(ms, ds, ps.x, ps.y, k);
    md_merge(mt, dt, pt.x, pt.y, k);
  }
  wave_md(ms, ds, k);
  wave_md(mt, dt, k);
  for (int s = lane; s < a.S; s += 64)
    a.stats[row * a.S + s] = s == 0 ? make_float4(ms, ds, mt, dt)
                                    : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
}

__global__ __launch_bounds__(64) void jsd_row_loss_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  if (threadIdx.x == 0) {
    const float2* lg = a.lg + row * a.S;
    float acc = lg[0].x;
    for (int j = 1; j < a.S; ++j) acc += lg[j].x;
    a.row_loss[row] = acc * a.row_scale;
  }
}

constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void loss_reduce_kernel(const float* row_loss,
                                                                     int64_t n, float scale,
                                                                     float* loss) {
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kReduceThreads) acc += row_loss[i];
  __shared__ double sh[kReduceThreads];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kReduceThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = static_cast<float>(sh[0] * static_cast<double>(scale));
}

// Sum of K-split fp32 partials in split order, rounded once to the dtype.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits,
                                                            int64_t M, int64_t N, T* out,
                                                            int64_t ldo) {
  const int64_t total4 = M * N / 4;
  const int64_t plane = M * N;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t e = i * 4;
    float4 acc = *reinterpret_cast<const float4*>(part + e);
    for (int s = 1; s < splits; ++s) {
      const float4 o = *reinterpret_cast<const float4*>(part + s * plane + e);
      acc.x += o.x;
      acc.y += o.y;
      acc.z += o.z;
      acc.w += o.w;
    }
    const int64_t m = e / N;
    const int64_t c = e % N;   // N is a multiple of 4, so all four share row m
    T* o = out + m * ldo + c;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<float4*>(o) = acc;
    } else {
      uint2 q;
      q.x = pack_bf16x2(acc.x, acc.y);
      q.y = pack_bf16x2(acc.z, acc.w);
      *reinterpret_cast<uint2*>(o) = q;
    }
  }
}

template <typename T>
hipError_t launch_loss_t(const JsdArgs& a, hipStream_t s, dim3 grid) {
  const dim3 block(kThreads);
  if (a.mode == kModeForwardKL)
    hipLaunchKernelGGL((jsd_loss_kernel<T, kModeForwardKL>), grid, block, 0, s, a);
  else if (a.mode == kModeReverseKL)
    hipLaunchKernelGGL((jsd_loss_kernel<T, kModeReverseKL>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((jsd_loss_kernel<T, kModeGeneralized>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Pass 2 when pass 3 computes the loss (bf16, generalized branch): only the
// cross-column sum G = sum_v g per (row, slice), into lg[.].y (lg[.].x = 0);
// the loss, which needs the accurate small-t form of r, is summed in pass 3.
__global__ __launch_bounds__(kThreads) void jsd_gsum_kernel(JsdArgs a) {
  const int64_t row = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_w;
  const int64_t v1 = min(a.V, v0 + a.slice_w);
  const uint16_t* zs = static_cast<const uint16_t*>(a.zs) + row * a.ld;
  const uint16_t* zt = static_cast<const uint16_t*>(a.zt) + row * a.ld;
  const float4 L = row_log_norms(a, row);
  const float k = a.k2;
  const float cg = -(1.f - a.beta) * kLn2;
  const GenRow rw = gen_row(L, 0.f, 0.f);  // a_s, a_t as in jsd_loss_kernel
  float gsum = 0.f;
  for (int64_t v = v0 + threadIdx.x * 8; v < v1; v += kThreads * 8) {
    const int n = static_cast<int>(min<int64_t>(8, v1 - v));
    float ys[8], yt[8];
    load8(zs, v, n, a.vec_ok, ys);
    load8(zt, v, n, a.vec_ok, yt);
    // Columns past the row end load as -inf in both rows: a tie, adding 0.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float as = gen_as(ys[i], k, rw), at = gen_at(yt[i], k, rw);
      gsum = gsum_plain(gsum, as, at, hw_exp2(as), a.beta, cg);
    }
  }
  gsum = wave_sum(gsum);
  __shared__ float sh[kWaves];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wave] = gsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = sh[0];
    for (int w = 1; w < kWaves; ++w) acc += sh[w];
    a.lg[row * a.S + s] = make_float2(0.f, acc);
  }
}

// Pass 3 over 64-row x 64-column tiles, bf16: dZ written in place as by
// jsd_grad_kernel, and the same tile, transposed through LDS, to
// dzt [V, ldt] for the weight-gradient product. A workgroup covers 64 rows and
// `span` columns (grad_t_span); threads 0..63 first merge their row's
// statistics and pass-2 partials. In the LDS tile, 16-byte chunk c of row r
// sits at c ^ ((r / 8) % 8), so both the row-wise writes and the column-wise
// reads are free of bank conflicts; two tile buffers alternate, so one
// barrier per tile suffices (a buffer is rewritten only after every thread
// has passed the barrier that follows its last read).
// LOSS (generalized and forward KL): the per-element loss terms are summed
// here instead of in pass 2, per row over the workgroup's columns, into
// lpart [column block][rows]; jsd_row_loss_merge_kernel adds them up.
template <int MODE, bool LOSS>
__global__ __launch_bounds__(kThreads) void jsd_grad_t_kernel(JsdArgs a, uint16_t* dzt,
                                                             int64_t ldt, int64_t span) {
  __shared__ float4 sh_L[64];
  __shared__ float sh_G[64];
  __shared__ uint4 tile[2][64][8];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t c_begin = static_cast<int64_t>(blockIdx.x) * span;
  const int64_t c_end = min(a.V, c_begin + span);
  const int t = threadIdx.x;
  if (t < 64) {
    const int64_t row = r0 + t;
    float4 L = make_float4(0.f, 0.f, 0.f, 0.f);
    float G = 0.f;
    if (row < a.rows) {
      const float4* st = a.stats + row * a.S;
      float4 acc = st[0];
      for (int s = 1; s < a.S; ++s) {
        md_merge(acc.x, acc.y, st[s].x, st[s].y, a.k2);
        md_merge(acc.z, acc.w, st[s].z, st[s].w, a.k2);
      }
      L = make_float4(acc.x, hw_log2(acc.y), acc.z, hw_log2(acc.w));
      if (MODE != kModeForwardKL) {
        const float2* lg = a.lg + row * a.S;
        float2 sum = lg[0];
        for (int j = 1; j < a.S; ++j) {
          sum.x += lg[j].x;
          sum.y += lg[j].y;
        }
        G = sum.y;
        if (!LOSS && blockIdx.x == 0) a.row_loss[row] = sum.x * a.row_scale;
      }
    }
    sh_L[t] = L;
    sh_G[t] = G;
  }
  __syncthreads();
  const uint16_t* zs = static_cast<const uint16_t*>(a.zs);
  const uint16_t* zt = static_cast<const uint16_t*>(a.zt);
  uint16_t* gr = static_cast<uint16_t*>(a.grad);
  const float k = a.k2;
  const float beta = a.beta;
  // Row-major: thread -> (row, 8-column chunk) for rows t/8 and t/8 + 32.
  // Whole 16-byte groups of both rows (and of the next 64-column tile) are
  // loaded before any of this tile is computed: dZ goes over the student
  // logits in place, so the compiler would otherwise keep each row's loads
  // behind the previous row's stores. The tile hand-offs wait for LDS
  // traffic only, so the next tile's loads stay in flight across them.
  const int chunk = t % 8;
  auto full = [&](int64_t row, int64_t v) { return a.vec_ok && row < a.rows && v + 8 <= a.V; };
  auto fetch = [&](int64_t c0, uint4 (&qs)[2], uint4 (&qt)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = r0 + t / 8 + 32 * h;
      const int64_t v = c0 + chunk * 8;
      if (full(row, v)) {
        qs[h] = ld_stream(zs + row * a.ld + v);
        qt[h] = ld_stream(zt + row * a.ld + v);
      }
    }
  };
  float lsum[2] = {0.f, 0.f};
  constexpr bool kGen = MODE == kModeGeneralized;
  const GenBeta gb = gen_beta(beta, a.grad_scale);
  // The dZ of 8 logits of one row, and its loss terms into *ls (for the
  // generalized branch, over ln 2).
  auto elem8 = [&](const uint4& qs, const uint4& qt, const float4& L, float G, const GenRow& rw,
                   float& ls) {
    const uint32_t ws[4] = {qs.x, qs.y, qs.z, qs.w};
    const uint32_t wt[4] = {qt.x, qt.y, qt.z, qt.w};
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float zsv = (i & 1) ? bf16_hi(ws[i >> 1]) : bf16_lo(ws[i >> 1]);
      const float ztv = (i & 1) ? bf16_hi(wt[i >> 1]) : bf16_lo(wt[i >> 1]);
      float l = 0.f;
      if constexpr (kGen) {
        gen_terms(gen_as(zsv, k, rw), gen_at(ztv, k, rw), rw.nG, gb, out[i], l);
      } else {
        const float as = (zsv - L.x) * k - L.y, at = (ztv - L.z) * k - L.w;
        float Q, P, g, gacc;
        jsd_terms<MODE>(as, at, beta, Q, P, l, g, gacc);
        out[i] = ((MODE == kModeForwardKL) ? (Q - P) : (g - Q * G)) * a.grad_scale;
      }
      if constexpr (LOSS) ls += l;
    }
    return make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]),
                      pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
  };
  // Interior workgroups (64 whole rows, every column tile whole, 16-byte
  // rows): a loop with no bounds checks over pointers advanced per tile.
  const bool interior = a.vec_ok && r0 + 64 <= a.rows && c_end - c_begin == span;
  if (interior) {
    const int rl0 = t / 8;
    const int64_t off0 = (r0 + rl0) * a.ld + c_begin + chunk * 8;
    const int64_t off1 = off0 + 32 * a.ld;
    const float4 L0 = sh_L[rl0], L1 = sh_L[rl0 + 32];
    const float G0 = sh_G[rl0], G1 = sh_G[rl0 + 32];
    const GenRow R0 = gen_row(L0, G0, a.grad_scale), R1 = gen_row(L1, G1, a.grad_scale);
    const int j = t % 8;
    uint16_t* d0 = dzt + (c_begin + rl0) * ldt + r0 + 8 * j;   // column c_begin + t/8
    uint16_t* d1 = d0 + 32 * ldt;                              // column c_begin + t/8 + 32
    const int ntile = static_cast<int>(span / 64);
    // q = (student row 0, student row 1, teacher row 0, teacher row 1) of
    // one tile. Two register sets alternate: the next tile's loads go to the
    // set not being computed, so nothing is copied between them.
    auto load_tile = [&](int it, uint4 (&q)[4]) {
      const int64_t c = static_cast<int64_t>(it) * 64;
      q[0] = ld_stream(zs + off0 + c);
      q[1] = ld_stream(zs + off1 + c);
      q[2] = ld_stream(zt + off0 + c);
      q[3] = ld_stream(zt + off1 + c);
    };
    auto do_tile = [&](int it, const uint4 (&q)[4]) {
      const int64_t c = static_cast<int64_t>(it) * 64;
      const uint4 p0 = elem8(q[0], q[2], L0, G0, R0, lsum[0]);
      const uint4 p1 = elem8(q[1], q[3], L1, G1, R1, lsum[1]);
      st_stream(gr + off0 + c, p0);
      st_stream(gr + off1 + c, p1);
      tile[it & 1][rl0][chunk ^ ((rl0 >> 3) & 7)] = p0;
      tile[it & 1][rl0 + 32][chunk ^ (((rl0 + 32) >> 3) & 7)] = p1;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const uint16_t* t16 = reinterpret_cast<const uint16_t*>(&tile[it & 1][0][0]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cl = rl0 + 32 * h;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int rl = 8 * j + i;
          e[i] = t16[rl * 64 + ((cl >> 3) ^ ((rl >> 3) & 7)) * 8 + (cl & 7)];
        }
        st_stream((h ? d1 : d0) + c * ldt,
                  make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                             e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)));
      }
    };
    uint4 qa[4], qb[4];
    load_tile(0, qa);
    for (int it = 0; it < ntile; it += 2) {
      if (it + 1 < ntile) load_tile(it + 1, qb);
      do_tile(it, qa);
      if (it + 1 >= ntile) break;
      if (it + 2 < ntile) load_tile(it + 2, qa);
      do_tile(it + 1, qb);
    }
  }
  uint4 cs[2], ct[2], ns[2], nt[2];
  if (!interior) fetch(c_begin, cs, ct);
  int buf = 0;
  for (int64_t c0 = interior ? c_end : c_begin; c0 < c_end; c0 += 64) {
    if (c0 + 64 < c_end) fetch(c0 + 64, ns, nt);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = t / 8 + 32 * h;
      const int64_t row = r0 + rl;
      const int64_t v = c0 + chunk * 8;
      uint4 packed = make_uint4(0, 0, 0, 0);
      if (row < a.rows && v < a.V) {
        const int n = static_cast<int>(min<int64_t>(8, a.V - v));
        const float4 L = sh_L[rl];
        const float G = sh_G[rl];
        float ys[8], yt[8], out[8];
        if (full(row, v)) {
          const uint32_t ws[4] = {cs[h].x, cs[h].y, cs[h].z, cs[h].w};
          const uint32_t wt[4] = {ct[h].x, ct[h].y, ct[h].z, ct[h].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ys[2 * e] = bf16_lo(ws[e]);
            ys[2 * e + 1] = bf16_hi(ws[e]);
            yt[2 * e] = bf16_lo(wt[e]);
            yt[2 * e + 1] = bf16_hi(wt[e]);
          }
        } else {
          load8(zs + row * a.ld, v, n, a.vec_ok, ys);
          load8(zt + row * a.ld, v, n, a.vec_ok, yt);
        }
        const GenRow rw = gen_row(L, G, a.grad_scale);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float l = 0.f;
          if constexpr (kGen) {
            gen_terms(gen_as(ys[i], k, rw), gen_at(yt[i], k, rw), rw.nG, gb, out[i], l);
          } else {
            const float as = (ys[i] - L.x) * k - L.y, at = (yt[i] - L.z) * k - L.w;
            float Q, P, g, gacc;
            jsd_terms<MODE>(as, at, beta, Q, P, l, g, gacc);
            out[i] = ((MODE == kModeForwardKL) ? (Q - P) : (g - Q * G)) * a.grad_scale;
          }
          // Columns past the row end load as -inf: no loss term (the
          // generalized one is NaN there).
          if constexpr (LOSS) lsum[h] += i < n ? l : 0.f;
        }
        packed = pack8_bf16(out, n);
        store8_packed(gr + row * a.ld, v, n, a.vec_ok, packed);
      }
      tile[buf][rl][chunk ^ ((rl >> 3) & 7)] = packed;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // Transposed: thread -> (column, eight consecutive rows); a wave writes
    // 8 rows of dzt, 128 contiguous bytes each.
    const uint16_t* t16 = reinterpret_cast<const uint16_t*>(&tile[buf][0][0]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cl = t / 8 + 32 * h;
      const int j = t % 8;
      const int64_t v = c0 + cl;
      const int64_t r = r0 + 8 * j;
      if (v < a.V && r < a.rows) {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int rl = 8 * j + i;
          e[i] = t16[rl * 64 + ((cl >> 3) ^ ((rl >> 3) & 7)) * 8 + (cl & 7)];
        }
        uint16_t* q = dzt + v * ldt + r;
        if (r + 8 <= a.rows) {
          st_stream(q, make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                                  e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)));
        } else {
          for (int i = 0; i < 8; ++i)
            if (r + i < a.rows) q[i] = e[i];
        }
      }
    }
    buf ^= 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cs[h] = ns[h];
      ct[h] = nt[h];
    }
  }
  if constexpr (LOSS) {
    // The 8 threads of a row are 8 consecutive lanes: sum them, fixed order
    // per lane pattern, and write this workgroup's partial of each row.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x = kGen ? lsum[h] * kLn2 : lsum[h];
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      const int64_t row = r0 + t / 8 + 32 * h;
      if (chunk == 0 && row < a.rows) a.lpart[static_cast<int64_t>(blockIdx.x) * a.rows + row] = x;
    }
  }
}

// Row losses from pass 3's per-workgroup partials: one wave per row, lane l
// adding blocks l, l + 64, ... in order, then a fixed butterfly over the
// lanes (the same order every run).
__global__ __launch_bounds__(256) void jsd_row_loss_merge_kernel(const float* lpart, int64_t rows,
                                                                 int nblk, float row_scale,
                                                                 float* row_loss) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int b = lane; b < nblk; b += 64) acc += lpart[static_cast<int64_t>(b) * rows + row];
  acc = wave_sum(acc);
  if (lane == 0) row_loss[row] = acc * row_scale;
}

template <typename T>
hipError_t launch_grad_t(const JsdArgs& a, hipStream_t s, dim3 grid) {
  const dim3 block(kThreads);
  if (a.mode == kModeForwardKL)
    hipLaunchKernelGGL((jsd_grad_kernel<T, kModeForwardKL>), grid, block, 0, s, a);
  else if (a.mode == kModeReverseKL)
    hipLaunchKernelGGL((jsd_grad_kernel<T, kModeReverseKL>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((jsd_grad_kernel<T, kModeGeneralized>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_jsd_stats(const JsdArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  if (dtype == 1)
    hipLaunchKernelGGL(jsd_stats_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(jsd_stats_kernel<float>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_jsd_loss(const JsdArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  return dtype == 1 ? launch_loss_t<uint16_t>(a, s, grid) : launch_loss_t<float>(a, s, grid);
}

hipError_t launch_jsd_grad(const JsdArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  return dtype == 1 ? launch_grad_t<uint16_t>(a, s, grid) : launch_grad_t<float>(a, s, grid);
}

hipError_t launch_jsd_grad_transposed(const JsdArgs& a, void* dzt, int64_t ldt, bool loss_in_pass3,
                                      hipStream_t s) {
  int64_t span = 0, nblk = 0;
  grad_t_geometry(a.rows, a.V, &span, &nblk);
  const int64_t row_blocks = (a.rows + 63) / 64;
  const dim3 grid(static_cast<unsigned>(nblk), static_cast<unsigned>(row_blocks));
  uint16_t* d = static_cast<uint16_t*>(dzt);
  const dim3 block(kThreads);
  if (loss_in_pass3 && a.mode == kModeForwardKL)
    hipLaunchKernelGGL((jsd_grad_t_kernel<kModeForwardKL, true>), grid, block, 0, s, a, d, ldt, span);
  else if (loss_in_pass3 && a.mode == kModeGeneralized)
    hipLaunchKernelGGL((jsd_grad_t_kernel<kModeGeneralized, true>), grid, block, 0, s, a, d, ldt, span);
  else if (a.mode == kModeForwardKL)
    hipLaunchKernelGGL((jsd_grad_t_kernel<kModeForwardKL, false>), grid, block, 0, s, a, d, ldt, span);
  else if (a.mode == kModeReverseKL)
    hipLaunchKernelGGL((jsd_grad_t_kernel<kModeReverseKL, false>), grid, block, 0, s, a, d, ldt, span);
  else
    hipLaunchKernelGGL((jsd_grad_t_kernel<kModeGeneralized, false>), grid, block, 0, s, a, d, ldt, span);
  return hipGetLastError();
}

hipError_t launch_jsd_gsum(const JsdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.S));
  hipLaunchKernelGGL(jsd_gsum_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_jsd_row_loss_merge(const JsdArgs& a, hipStream_t s) {
  int64_t span = 0, nblk = 0;
  grad_t_geometry(a.rows, a.V, &span, &nblk);
  const dim3 grid(static_cast<unsigned>((a.rows + 3) / 4));
  hipLaunchKernelGGL(jsd_row_loss_merge_kernel, grid, dim3(256), 0, s, a.lpart, a.rows,
                     static_cast<int>(nblk), a.row_scale, a.row_loss);
  return hipGetLastError();
}

hipError_t launch_jsd_stats_merge(const JsdArgs& a, const float2* part_s, const float2* part_t,
                                  int64_t tiles, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.rows + 3) / 4));
  hipLaunchKernelGGL(jsd_stats_merge_kernel, grid, dim3(256), 0, s, a, part_s, part_t, tiles);
  return hipGetLastError();
}

hipError_t launch_jsd_row_loss(const JsdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(jsd_row_loss_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(64), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* row_loss, int64_t n, float scale, float* loss,
                              hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, s, row_loss, n,
                     scale, loss);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, void* out,
                                int64_t ldo, int dtype, hipStream_t s) {
  const int64_t total4 = M * N / 4;
  const int64_t blocks = std::min<int64_t>((total4 + 255) / 256, 256 * 16);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (dtype == 1)
    hipLaunchKernelGGL(splitk_reduce_kernel<uint16_t>, grid, dim3(256), 0, s, part, splits, M,
                       N, static_cast<uint16_t*>(out), ldo);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, grid, dim3(256), 0, s, part, splits, M, N,
                       static_cast<float*>(out), ldo);
  return hipGetLastError();
}

}  // namespace fljsd
