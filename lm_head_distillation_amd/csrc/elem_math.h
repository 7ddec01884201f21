// fp32 element math shared by the loss kernels: hardware transcendentals,
// 8-wide row loads and stores with bf16 conversion, wave sums, expm1 / log1p
// with full relative accuracy, the mixture log ln(w e^x + 1 - w) built on
// them, and the Bregman-term series of the KL branches.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace fljsd {

constexpr float kLn2 = 0.693147180559945309f;

__device__ inline float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ inline float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even and packed as bf16, a in the low
// half: one gfx950 v_cvt_pk_bf16_f32. It agrees bit for bit with
// round-to-nearest-even on every non-NaN input (all 2^32 fp32 patterns were
// compared on the device, denormals included); a NaN stays a NaN.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ inline uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte load and store for data a pass touches once (the
// logits streamed by the loss passes, the gradients they write): on MI355X a
// plain copy moves 5.3 TB/s, one with non-temporal loads and stores 5.7. The
// 8-element helpers below stream by default; the cross-entropy passes, whose
// second pass re-reads what the first read (partly still in the Infinity
// Cache at small chunks), measured faster with plain accesses.
__device__ inline uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void st_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4_t*>(p));
}

// Eight values as packed bf16; entries at or past n are zero.
__device__ inline uint4 pack8_bf16(const float* x, int n) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = i < n ? x[i] : 0.f;
  return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                    pack_bf16x2(y[6], y[7]));
}

// Load up to 8 consecutive elements starting at column v; lanes at or past n
// read as `fill` (-inf for logits: a masked column carries no probability
// mass). A full group uses 16-byte loads when `vec` says the rows are 16-byte
// aligned.
template <bool STREAM = true>
__device__ inline void load8(const float* p, int64_t v, int n, bool vec, float* x,
                             float fill = -INFINITY) {
  if (n == 8 && vec) {
    const uint4 a = STREAM ? ld_stream(p + v) : *reinterpret_cast<const uint4*>(p + v);
    const uint4 b = STREAM ? ld_stream(p + v + 4) : *reinterpret_cast<const uint4*>(p + v + 4);
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = i < n ? p[v + i] : fill;
  }
}

template <bool STREAM = true>
__device__ inline void load8(const uint16_t* p, int64_t v, int n, bool vec, float* x,
                             float fill = -INFINITY) {
  if (n == 8 && vec) {
    const uint4 q = STREAM ? ld_stream(p + v) : *reinterpret_cast<const uint4*>(p + v);
    x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x);
    x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
    x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z);
    x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = i < n ? __uint_as_float(uint32_t(p[v + i]) << 16) : fill;
  }
}

template <bool STREAM = true>
__device__ inline void store16(void* p, uint4 v) {
  if (STREAM)
    st_stream(p, v);
  else
    *static_cast<uint4*>(p) = v;
}

template <bool STREAM = true>
__device__ inline void store8(float* p, int64_t v, int n, bool vec, const float* x) {
  if (n == 8 && vec) {
    store16<STREAM>(p + v, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                      __float_as_uint(x[2]), __float_as_uint(x[3])));
    store16<STREAM>(p + v + 4, make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]),
                                          __float_as_uint(x[6]), __float_as_uint(x[7])));
  } else {
    for (int i = 0; i < n; ++i) p[v + i] = x[i];
  }
}

// Up to 8 packed bf16 values (pack8_bf16) to columns v .. v + n - 1.
template <bool STREAM = true>
__device__ inline void store8_packed(uint16_t* p, int64_t v, int n, bool vec, uint4 q) {
  if (n == 8 && vec) {
    store16<STREAM>(p + v, q);
  } else {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    for (int i = 0; i < n; ++i) p[v + i] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
  }
}

template <bool STREAM = true>
__device__ inline void store8(uint16_t* p, int64_t v, int n, bool vec, const float* x) {
  store8_packed<STREAM>(p, v, n, vec, pack8_bf16(x, n));
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// expm1(x) for |x| <= 80, either sign (xt = x / ln 2): the degree-9 Taylor
// polynomial below |x| = 1/2, 2^xt - 1 beyond (e^x >= 1.65 or <= 0.61 there,
// so the subtraction costs at most a few ulp).
__device__ inline float expm1_f32(float x, float xt) {
  float p = 1.f / 362880.f;
  p = fmaf(p, x, 1.f / 40320.f);
  p = fmaf(p, x, 1.f / 5040.f);
  p = fmaf(p, x, 1.f / 720.f);
  p = fmaf(p, x, 1.f / 120.f);
  p = fmaf(p, x, 1.f / 24.f);
  p = fmaf(p, x, 1.f / 6.f);
  p = fmaf(p, x, 0.5f);
  p = fmaf(p, x, 1.f);
  return fabsf(x) < 0.5f ? p * x : hw_exp2(xt) - 1.f;
}

// log1p(y) for y >= -1/2: the atanh series for |y| <= 1/4, the hardware log2
// of 1 + y beyond (1 + y then lies in [1/2, 3/4] or above 5/4).
__device__ inline float log1p_f32(float y) {
  const float s = y * hw_rcp(2.f + y);
  const float s2 = s * s;
  float p = 1.f / 11.f;
  p = fmaf(p, s2, 1.f / 9.f);
  p = fmaf(p, s2, 1.f / 7.f);
  p = fmaf(p, s2, 1.f / 5.f);
  p = fmaf(p, s2, 1.f / 3.f);
  p = fmaf(p, s2, 1.f);
  return fabsf(y) <= 0.25f ? 2.f * s * p : hw_log2(1.f + y) * kLn2;
}

// Mixture weights of the fp32 gradient terms: for a reference log-ratio
// D_c = tc ln 2 (tc in base 2), w = beta e^Dc / (beta e^Dc + 1 - beta) and
// cw = 1 - w, each to full relative accuracy, with lw = ln w and lc = ln cw
// finite even where w or cw underflows.
struct MixWeights {
  float w, cw, lw, lc;
};
__device__ inline MixWeights mix_weights(float tc, float beta) {
  const float cb = 1.f - beta;
  const bool neg = tc < 0.f;
  const float E = hw_exp2(-fabsf(tc));
  const float den = neg ? fmaf(beta, E, cb) : fmaf(cb, E, beta);
  const float rden = 1.f / den;
  const float lden = hw_log2(den) * kLn2;
  const float dabs = fabsf(tc) * kLn2;
  MixWeights m;
  m.w = (neg ? beta * E : beta) * rden;
  m.cw = (neg ? cb : cb * E) * rden;
  m.lw = hw_log2(beta) * kLn2 - (neg ? dabs : 0.f) - lden;
  m.lc = hw_log2(cb) * kLn2 - (neg ? 0.f : dabs) - lden;
  return m;
}

// rho(x) = ln(w e^x + cw) for the weights above (xt = x / ln 2), with full
// relative accuracy at every x: log1p(w expm1(x)) while w expm1(x) >= -1/2
// (no cancellation in the argument or the result), the direct log of the two
// positive terms below that (the result is then below ln(1/2)), and beyond
// |x| = 80 the log-sum-exp of ln w + x and ln cw.
__device__ inline float mix_log(float x, float xt, const MixWeights& m) {
  const float xc = fminf(fmaxf(x, -80.f), 80.f);
  const float xtc = fminf(fmaxf(xt, -115.f), 115.f);
  const float y = m.w * expm1_f32(xc, xtc);
  const float r_near = y >= -0.5f ? log1p_f32(y) : hw_log2(fmaf(m.w, hw_exp2(xtc), m.cw)) * kLn2;
  const float s = x + m.lw;
  const float hi = fmaxf(s, m.lc), lo = fminf(s, m.lc);
  const float r_far = hi + log1p_f32(hw_exp2((lo - hi) * 1.4426950408889634f));
  return fabsf(x) > 80.f ? r_far : r_near;
}

// Weights of the fp32 generalized terms: (beta, 1 - beta) for r = ln(beta
// e^D + 1 - beta), and the mirrored pair for D - r = -ln((1 - beta) e^-D +
// beta), both evaluated by mix_log.
struct BetaWeights {
  MixWeights r, dmr;
};
__device__ inline BetaWeights beta_weights(float beta) {
  return {mix_weights(0.f, beta), mix_weights(0.f, 1.f - beta)};
}

// r = ln(beta e^D + 1 - beta) and D - r for 0 < beta < 1, from bf16 inputs;
// t = D / ln 2. Away from D = 0, r = ln u + max(D, 0) with
// u = c e^(-|D|) + 1 - c (c = beta for D < 0, else 1 - beta): u lies in
// [min(beta, 1 - beta), 1], so nothing overflows, and rounding u costs r an
// absolute ~4e-8. u is evaluated as 1 - c (1 - e^(-|D|)), exactly 1 at
// D = 0 whatever the rounding of 1 - beta (beta + (1 - beta) is not 1 in
// fp32 for most beta, a bias of the same sign at every element otherwise).
// Near D = 0, where rounding u would be a large relative error of a
// small r, r is r(D)'s Taylor series instead: r is the cumulant generating
// function of a Bernoulli(beta) variable, so the coefficient of D^n / n! is
// that variable's n-th cumulant. The series runs to degree 4 below |D| = 1/16
// (truncation below 1.3e-7 relative there).
__device__ inline void jsd_r_direct(float D, float t, float beta, float& r, float& dmr) {
  const bool neg = D < 0.f;
  const float e = hw_exp2(-fabsf(t));
  const float L1 = hw_log2(fmaf(-(neg ? beta : 1.f - beta), 1.f - e, 1.f)) * kLn2;
  const float v = beta * (1.f - beta);  // the Bernoulli variance
  float p = v * (1.f - 6.f * v) * (1.f / 24.f);
  p = fmaf(p, D, v * (1.f - 2.f * beta) * (1.f / 6.f));
  p = fmaf(p, D, 0.5f * v);
  p = fmaf(p, D, beta);
  const float rs = p * D;
  const bool small = fabsf(D) < 0.0625f;
  r = small ? rs : (neg ? L1 : D + L1);
  dmr = small ? D - rs : (neg ? D - L1 : -L1);
}

// D e^D - expm1(D) for |D| < 1/4: sum over k >= 2 of (k-1) D^k / k!.
__device__ inline float kl_fwd_series(float D) {
  float p = 1.f / 5760.f;
  p = fmaf(p, D, 1.f / 840.f);
  p = fmaf(p, D, 1.f / 144.f);
  p = fmaf(p, D, 1.f / 30.f);
  p = fmaf(p, D, 1.f / 8.f);
  p = fmaf(p, D, 1.f / 3.f);
  p = fmaf(p, D, 0.5f);
  return p * D * D;
}

// expm1(D) - D for |D| < 1/4: sum over k >= 2 of D^k / k!.
__device__ inline float kl_rev_series(float D) {
  float p = 1.f / 40320.f;
  p = fmaf(p, D, 1.f / 5040.f);
  p = fmaf(p, D, 1.f / 720.f);
  p = fmaf(p, D, 1.f / 120.f);
  p = fmaf(p, D, 1.f / 24.f);
  p = fmaf(p, D, 1.f / 6.f);
  p = fmaf(p, D, 0.5f);
  return p * D * D;
}

// Merge of two (max, denominator) pairs; maxima in logit units, denominators
// in base 2 with scale k. Commutative bit for bit (max and a two-term IEEE
// sum are), so both butterfly partners agree. The multiply-adds are written
// as explicit fmaf: the compiler may otherwise contract either product into
// the sum, differently at different call sites, and equal inputs (a teacher
// identical to the student) must give bit-identical statistics.
__device__ inline void md_merge(float& m, float& d, float mo, float dof, float k) {
  const float M = fmaxf(m, mo);
  if (M == -INFINITY) {
    m = -INFINITY;
    d = 0.f;
    return;
  }
  const float a = d * hw_exp2((m - M) * k);
  const float b = dof * hw_exp2((mo - M) * k);
  d = fmaxf(a, b) + fminf(a, b);
  m = M;
}

// Fold 8 logits into a running (max, denominator).
__device__ inline void md_update8(float& m, float& d, const float* z, float k) {
  float mx = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
  if (mx == -INFINITY) return;
  float acc = 0.f;
  const float mn = fmaxf(m, mx);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += hw_exp2((z[i] - mn) * k);
  d = fmaf(d, hw_exp2((m - mn) * k), acc);
  m = mn;
}

__device__ inline void wave_md(float& m, float& d, float k) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o, 64);
    const float dof = __shfl_xor(d, o, 64);
    md_merge(m, d, mo, dof, k);
  }
}

}  // namespace fljsd
